"""The single poly-update launch of small calls whose matrices all have
m <= 256, against the two-launch path (poly, then update).  The matrices of
a call are independent, so a matrix computed alone (one launch per
iteration: no poly launch is timed) and beside a 512 x 512 matrix (two
launches: five poly launches are timed) must agree bit for bit; both match
the oracle."""
import numpy as np
import pytest

from gpu_helpers import BETA, COEFFS, LR, NS_TOL, bf16_gpu, bf16_to_np, empty_bf16, rel_f, say, to_gpu, torch_mod
from oracle import muon_oracle as om

pytestmark = pytest.mark.gpu

KERNEL_POLY = 3  # MUON_KERNEL_POLY
COMPANION = (512, 512)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import optimizer_muon_step_amd as mu
    mu._lib.load()
    yield
    torch.cuda.synchronize()


def _rand_bf16(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x /= np.float32(np.linalg.norm(x.astype(np.float64)) + 1e-7)
    return om.bf16_bits(x)


def _ns_bits(shapes, bits):
    """Newton-Schulz outputs (uint16 bits) of one call, and the number of
    poly launches it made."""
    import optimizer_muon_step_amd as mu
    torch = torch_mod()
    xs = [bf16_gpu(b) for b in bits]
    outs = [empty_bf16(s) for s in shapes]
    mu.muon_timing_enable(KERNEL_POLY)
    try:
        mu.muon_newton_schulz(xs, outs, 5, COEFFS)
        torch.cuda.synchronize()
        _, polys = mu.muon_timing_read()
    finally:
        mu.muon_timing_enable(-1)
    return [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs], polys


FUSED_SHAPES = [(256, 512), (100, 300), (512, 200), (129, 257), (1, 7), (256, 1024), (64, 64)]


@pytest.mark.parametrize("shape", FUSED_SHAPES)
def test_one_launch_matches_two_launches_bit_for_bit(shape):
    say(f"[fused ns] shape={shape}")
    bits = _rand_bf16(shape, 500 + shape[0] + 3 * shape[1])
    comp = _rand_bf16(COMPANION, 77)
    (alone,), polys_alone = _ns_bits([shape], [bits])
    (beside, _), polys_beside = _ns_bits([shape, COMPANION], [bits, comp])
    say(f"  poly launches: alone {polys_alone}, beside {COMPANION} {polys_beside}")
    assert polys_alone == 0 and polys_beside == 5
    assert np.array_equal(alone, beside)
    X0 = om.bf16_to_f32(bits)
    Xc, tr = om.canonical(X0)
    want = om.newton_schulz(np.ascontiguousarray(Xc), 5, COEFFS)
    want = want.T if tr else want
    e = rel_f(om.bf16_to_f32(alone), want)
    say(f"  relF {e:.3e}")
    assert e <= NS_TOL


def test_several_matrices_in_one_launch():
    """A fused call of several shapes: each matrix's bits equal its result
    from a two-launch call."""
    shapes = [(256, 512), (100, 300), (512, 200), (3, 256)]
    bits = [_rand_bf16(s, 900 + i) for i, s in enumerate(shapes)]
    together, polys = _ns_bits(shapes, bits)
    assert polys == 0
    comp = _rand_bf16(COMPANION, 78)
    for s, b, t in zip(shapes, bits, together):
        (ref, _), p2 = _ns_bits([s, COMPANION], [b, comp])
        assert p2 == 5
        assert np.array_equal(t, ref), f"{s}"


def test_fused_step_matches_two_launch_step():
    """The whole step (momentum, cast, NS, apply) on a 256 x 512 matrix, alone
    and beside a 512 x 512 one, two steps: W, momentum and the bf16 updates
    agree bit for bit."""
    import optimizer_muon_step_amd as mu
    torch = torch_mod()
    rng = np.random.default_rng(4242)
    W0 = (rng.standard_normal((256, 512)) * 0.02).astype(np.float32)
    G = [(rng.standard_normal((256, 512)) * 1e-3).astype(np.float32) for _ in range(2)]
    Wc0 = (rng.standard_normal(COMPANION) * 0.02).astype(np.float32)
    Gc = [(rng.standard_normal(COMPANION) * 1e-3).astype(np.float32) for _ in range(2)]
    res = []
    for with_comp in (False, True):
        W = [to_gpu(W0)] + ([to_gpu(Wc0)] if with_comp else [])
        M = [torch.zeros_like(w) for w in W]
        for s in range(2):
            Gs = [to_gpu(G[s])] + ([to_gpu(Gc[s])] if with_comp else [])
            U = [empty_bf16(w.shape) for w in W]
            mu.muon_step(W, Gs, M, LR, BETA, 5, COEFFS, updates=U)
        torch.cuda.synchronize()
        res.append((W[0].cpu().numpy(), M[0].cpu().numpy(), U[0].view(torch.int16).cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
