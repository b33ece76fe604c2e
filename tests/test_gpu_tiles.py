"""Tile shapes are chosen per call and per kernel kind (large, medium or
small tiles, from the call's tile counts), but every output element
accumulates its K in the same MFMA order whatever the tile, so a matrix's
result does not depend on the choice unless a long-K Gram tile is cut.  The
same matrices computed alone (medium or shallow small tiles) and inside a call whose
companions make every kind take the large tiles agree bit for bit; no Gram
tile is cut in either call."""
import numpy as np
import pytest

from gpu_helpers import COEFFS, NS_TOL, bf16_gpu, empty_bf16, rel_f, say, torch_mod
from oracle import muon_oracle as om

pytestmark = pytest.mark.gpu


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


def _ns_bits(bits):
    import optimizer_muon_step_amd as mu
    torch = torch_mod()
    xs = [bf16_gpu(b) for b in bits]
    outs = [empty_bf16(b.shape) for b in bits]
    mu.muon_newton_schulz(xs, outs, 5, COEFFS)
    torch.cuda.synchronize()
    return [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs]


# Eight 2048 x 2048 matrices: 288 Gram tiles of 256 (large, K 32 within
# twice the share of 36: not cut), 1088 poly tiles of 128 (large), 704
# update tiles of 192 x 256 in 3 rounds against 1024 of 128 x 256 in 4
# (large).
COMPANIONS = [(2048, 2048)] * 8


@pytest.mark.parametrize("shapes", [
    # Gram 128 x 128 (36 tiles of 256: fewer than the CUs; 136 of 128, K 32
    # within twice the share of 17), poly large (136 tiles of 128), update
    # on the small 64 x 128 tiles with the shallow ring (128 tiles of
    # 128 x 256 would leave half the CUs idle)
    [(2048, 2048)],
    # Gram and poly medium: Gram 108 tiles of 128 (K 16, share 8), poly 108
    # tiles of 128 (at most 128: 64 x 64 tiles); update on the shallow small
    # tiles (96 tiles of 128 x 256 would leave most CUs idle)
    [(1024, 1024)] * 3,
])
def test_medium_tiles_match_large_tiles_bit_for_bit(shapes):
    say(f"[tiles] {shapes} alone and beside {len(COMPANIONS)} x {COMPANIONS[0]}")
    bits = [_rand_bf16(s, 700 + 13 * i + s[0]) for i, s in enumerate(shapes)]
    comp = [_rand_bf16(s, 800 + i) for i, s in enumerate(COMPANIONS)]
    alone = _ns_bits(bits)
    beside = _ns_bits(bits + comp)[:len(shapes)]
    for s, a, b, x in zip(shapes, alone, beside, bits):
        assert np.array_equal(a, b), f"{s}"
        X0 = om.bf16_to_f32(x)
        want = om.newton_schulz(X0, 5, COEFFS)
        e = rel_f(om.bf16_to_f32(a), want)
        say(f"  {s}: relF {e:.3e}")
        assert e <= NS_TOL
