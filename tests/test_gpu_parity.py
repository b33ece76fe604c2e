"""GPU parity: the HIP library against the CPU oracle, element by element,
on the same seeded inputs.  Bars: Newton-Schulz outputs and parameter
updates within 1e-2 relative Frobenius error per matrix, fp32 momentum
buffers within 1e-6 (in practice bit-identical)."""
import math

import numpy as np
import pytest

from gpu_helpers import (BETA, COEFFS, LR, NS_TOL, bf16_gpu, bf16_to_np, check_matrix, empty_bf16, gpu_step,
                         oracle_steps, rel_f, say, to_gpu, torch_mod)
from oracle import muon_oracle as om
from optimizer_muon_step_amd import workloads as wl

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


NS_SHAPES = [(256, 512), (128, 128), (200, 300), (300, 200), (129, 1000), (1, 7), (7, 1), (1, 1), (384, 384),
             (64, 2304)]


@pytest.mark.parametrize("shape", NS_SHAPES)
@pytest.mark.parametrize("k", [1, 5])
def test_newton_schulz_core(shape, k):
    import optimizer_muon_step_amd as mu
    say(f"[ns core] shape={shape} k={k}")
    bits = _rand_bf16(shape, 17 + shape[0] * 7 + shape[1])
    x = bf16_gpu(bits)
    out = empty_bf16(shape)
    mu.muon_newton_schulz([x], [out], k, COEFFS)
    got = bf16_to_np(out)
    X0 = om.bf16_to_f32(bits)
    Xc, tr = om.canonical(X0)
    want = om.newton_schulz(np.ascontiguousarray(Xc), k, COEFFS)
    want = want.T if tr else want
    e = rel_f(got, want)
    say(f"  relF {e:.3e}  exact elements {np.mean(got == want):.4f}")
    assert got.shape == want.shape
    assert e <= (3e-3 if k == 1 else NS_TOL)


def test_newton_schulz_batched_mixed_shapes_in_place():
    """Several shapes in one call, output written over the input."""
    import optimizer_muon_step_amd as mu
    shapes = [(256, 512), (512, 256), (130, 130), (3, 500)]
    bits = [_rand_bf16(s, 100 + i) for i, s in enumerate(shapes)]
    xs = [bf16_gpu(b) for b in bits]
    mu.muon_newton_schulz(xs, xs, 5, COEFFS)
    for s, b, x in zip(shapes, bits, xs):
        X0 = om.bf16_to_f32(b)
        Xc, tr = om.canonical(X0)
        want = om.newton_schulz(np.ascontiguousarray(Xc), 5, COEFFS)
        want = want.T if tr else want
        e = rel_f(bf16_to_np(x), want)
        say(f"  {s}: relF {e:.3e}")
        assert e <= NS_TOL


def _monomial(n, m, rng, transpose):
    g = np.zeros((n, m), np.float32)
    cols = rng.permutation(m)[:n]
    g[np.arange(n), cols] = rng.integers(1, 8, n) * rng.choice([-1, 1], n)
    return g.T.copy() if transpose else g


@pytest.mark.parametrize("shape,transpose", [((12, 20), False), ((200, 300), False), ((130, 260), True),
                                             ((256, 256), False), ((40, 3000), False), ((300, 9000), True)])
def test_monomial_step_bit_exact(shape, transpose):
    """One non-zero per row and column: every dot product has one term, so the
    GPU must reproduce the oracle's storage points bit for bit."""
    say(f"[monomial] shape={shape} transpose={transpose}")
    rng = np.random.default_rng(shape[0] + 1000 * shape[1])
    g = _monomial(*shape, rng, transpose)
    W = rng.standard_normal(g.shape).astype(np.float32)
    m = {"W": W, "buf": np.zeros_like(W), "grads": [g]}
    Wg, Mg, Ug = gpu_step([m], "grads", 1)
    r = oracle_steps(m, 1)
    assert np.array_equal(Mg[0].cpu().numpy(), r["buf"])
    assert np.array_equal(bf16_to_np(Ug[0]), r["O"])
    assert np.array_equal(Wg[0].cpu().numpy(), r["W"])


# Long K.  A call with a Gram K of more than 32 slices is not small, and
# its long-K Gram tiles are cut into K chunks whose fp32 partials a reduce
# pass sums: a single ragged tile row (64 x 4100), diagonal tiles of 1024
# slices (256 x 65536), diagonal and off-diagonal tiles of a 1024-row
# matrix, and ragged tall ones; each of these runs the 128-wide Gram tiles.
@pytest.mark.parametrize("shape", [(64, 4100), (512, 20000), (20001, 300), (256, 65536), (1024, 20000),
                                   (20001, 600)])
def test_newton_schulz_long_k_split(shape):
    import optimizer_muon_step_amd as mu
    say(f"[ns long K] shape={shape}")
    bits = _rand_bf16(shape, 31 + shape[0] + shape[1])
    x = bf16_gpu(bits)
    out = empty_bf16(shape)
    mu.muon_newton_schulz([x], [out], 5, COEFFS)
    X0 = om.bf16_to_f32(bits)
    Xc, tr = om.canonical(X0)
    want = om.newton_schulz(np.ascontiguousarray(Xc), 5, COEFFS)
    want = want.T if tr else want
    e = rel_f(bf16_to_np(out), want)
    say(f"  relF {e:.3e}")
    assert e <= NS_TOL


def test_newton_schulz_long_k_mixed_with_short():
    import optimizer_muon_step_amd as mu
    shapes = [(1024, 20000), (256, 256), (300, 200), (64, 2304)]
    bits = [_rand_bf16(s, 200 + i) for i, s in enumerate(shapes)]
    xs = [bf16_gpu(b) for b in bits]
    outs = [empty_bf16(s) for s in shapes]
    mu.muon_newton_schulz(xs, outs, 5, COEFFS)
    for s, b, o in zip(shapes, bits, outs):
        X0 = om.bf16_to_f32(b)
        Xc, tr = om.canonical(X0)
        want = om.newton_schulz(np.ascontiguousarray(Xc), 5, COEFFS)
        want = want.T if tr else want
        e = rel_f(bf16_to_np(o), want)
        say(f"  {s}: relF {e:.3e}")
        assert e <= NS_TOL


def _run_config(name, steps=2, sample=None):
    specs = wl.config_specs(name)
    idx = list(range(len(specs)))
    mats = [wl.make_matrix(name, i, steps) for i in idx]
    say(f"[{name}] {len(mats)} matrices, {sum(s.rows * s.cols for s in specs)} params, {steps} steps")
    Wg, Mg, Ug = gpu_step(mats, "grads", steps)
    check = idx if sample is None else sample
    errs = []
    for i in check:
        r = oracle_steps(mats[i], steps)
        spec = specs[i]
        errs.append(check_matrix(f"{name}[{i}] {spec.rows}x{spec.cols} {spec.kind}", Wg[i], Mg[i], Ug[i], r,
                                 mats[i]["W"].astype(np.float64)))
    return errs


def test_step_c1():
    _run_config("c1", steps=2)


def test_step_c2():
    _run_config("c2", steps=2)


def test_step_c5():
    _run_config("c5", steps=1)


def test_step_c3_full():
    _run_config("c3", steps=1)


def test_step_c4_sampled():
    """1.47 B parameters in one launch sequence; the oracle checks one matrix
    of each shape, spread over the layers."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    name = "c4"
    specs = wl.config_specs(name)
    sample = [0, 1 + 4 * 17, 2 + 4 * 31, 3 + 4 * 47]
    say(f"[c4] generating {len(specs)} matrices on the host")
    W, M, G, W0 = [], [], [], {}
    for i, spec in enumerate(specs):
        w = wl.make_params(name, i, spec)
        if i in sample:
            W0[i] = w
        W.append(to_gpu(w))
        M.append(torch.zeros((spec.rows, spec.cols), dtype=torch.float32, device="cuda"))
        G.append(to_gpu(wl.make_grad(name, i, spec, 1)))
    U = [empty_bf16((s.rows, s.cols)) if i in sample else None for i, s in enumerate(specs)]
    say("[c4] running one step on the GPU")
    mu.muon_step(W, G, M, LR, BETA, 5, COEFFS, updates=U)
    torch.cuda.synchronize()
    del G
    for i in sample:
        spec = specs[i]
        m = {"W": W0[i], "buf": np.zeros((spec.rows, spec.cols), np.float32),
             "grads": [wl.make_grad(name, i, spec, 1)]}
        r = oracle_steps(m, 1)
        check_matrix(f"c4[{i}] {spec.rows}x{spec.cols}", W[i], M[i], U[i], r, W0[i].astype(np.float64))


def test_ns_steps_zero_applies_x0():
    rng = np.random.default_rng(5)
    m = {"W": rng.standard_normal((96, 160)).astype(np.float32), "buf": np.zeros((96, 160), np.float32),
         "grads": [rng.standard_normal((96, 160)).astype(np.float32)]}
    Wg, Mg, Ug = gpu_step([m], "grads", 1, ns_steps=0)
    r = oracle_steps(m, 1, ns_steps=0)
    # X0 = bf16(u * s): one rounding from identical fp32 inputs, same s
    assert np.array_equal(bf16_to_np(Ug[0]), r["O"])
    assert np.array_equal(Wg[0].cpu().numpy(), r["W"])


@pytest.mark.parametrize("shapes", [[(2048, 2048), (2048, 2049), (4097, 1024)]])
def test_norm_scale_on_both_sides_of_the_fold(shapes):
    """A matrix of at most 256 norm partials (16384 elements each) has its
    scale summed by every cast block, a larger one by the finalisation
    launch; 2048 x 2048 has exactly 256, 2048 x 2049 and the tall 4097 x 1024
    have 257.  With ns_steps = 0 the update is X0 = bf16(u * s), one rounding
    of identical fp32 inputs with the same s, so both paths must match the
    oracle bit for bit."""
    rng = np.random.default_rng(11)
    mats = [{"W": rng.standard_normal(s).astype(np.float32), "buf": (rng.standard_normal(s) * 1e-3).astype(np.float32),
             "grads": [(rng.standard_normal(s) * 1e-3).astype(np.float32)]} for s in shapes]
    say(f"[norm fold] {shapes}: {[-(-s[0] * s[1] // 16384) for s in shapes]} partials")
    Wg, Mg, Ug = gpu_step(mats, "grads", 1, ns_steps=0)
    for i, m in enumerate(mats):
        r = oracle_steps(m, 1, ns_steps=0)
        assert np.array_equal(Mg[i].cpu().numpy(), r["buf"])
        assert np.array_equal(bf16_to_np(Ug[i]), r["O"]), f"{shapes[i]}"
        assert np.array_equal(Wg[i].cpu().numpy(), r["W"]), f"{shapes[i]}"


def test_zero_gradient_leaves_params():
    W = np.random.default_rng(6).standard_normal((64, 128)).astype(np.float32)
    m = {"W": W, "buf": np.zeros_like(W), "grads": [np.zeros_like(W)]}
    Wg, Mg, Ug = gpu_step([m], "grads", 1)
    assert np.array_equal(Wg[0].cpu().numpy(), W)
    assert np.all(bf16_to_np(Ug[0]) == 0)


def test_nan_stays_in_its_matrix():
    rng = np.random.default_rng(7)
    a = {"W": rng.standard_normal((64, 96)).astype(np.float32), "buf": np.zeros((64, 96), np.float32),
         "grads": [rng.standard_normal((64, 96)).astype(np.float32)]}
    b = {"W": rng.standard_normal((64, 96)).astype(np.float32), "buf": np.zeros((64, 96), np.float32),
         "grads": [rng.standard_normal((64, 96)).astype(np.float32)]}
    b["grads"][0][3, 5] = np.nan
    Wg, Mg, Ug = gpu_step([a, b], "grads", 1)
    assert np.all(np.isfinite(Wg[0].cpu().numpy()))
    assert np.isnan(Wg[1].cpu().numpy()).any()
    r = oracle_steps(a, 1)
    assert rel_f(bf16_to_np(Ug[0]), r["O"]) <= NS_TOL


def test_ragged_and_degenerate_shapes_in_one_call():
    rng = np.random.default_rng(8)
    shapes = [(1, 1), (1, 300), (300, 1), (129, 257), (257, 129), (127, 127), (5, 4099)]
    mats = [{"W": rng.standard_normal(s).astype(np.float32), "buf": np.zeros(s, np.float32),
             "grads": [rng.standard_normal(s).astype(np.float32), rng.standard_normal(s).astype(np.float32)]}
            for s in shapes]
    Wg, Mg, Ug = gpu_step(mats, "grads", 2)
    for i, (s, m) in enumerate(zip(shapes, mats)):
        r = oracle_steps(m, 2)
        check_matrix(f"{s}", Wg[i], Mg[i], Ug[i], r, m["W"].astype(np.float64))


def test_deterministic_and_resumable():
    """Two runs are bit-identical, and stopping after one step, copying the
    state out and resuming matches running straight through."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    mats = [wl.make_matrix("c2", i, 3) for i in range(4)]
    W1, M1, _ = gpu_step(mats, "grads", 3, want_updates=False)
    W2, M2, _ = gpu_step(mats, "grads", 3, want_updates=False)
    for a, b in zip(W1 + M1, W2 + M2):
        assert torch.equal(a, b)
    # resume: one step, round-trip the state through the host, two more steps
    W = [to_gpu(m["W"]) for m in mats]
    M = [to_gpu(m["buf"]) for m in mats]
    mu.muon_step(W, [to_gpu(m["grads"][0]) for m in mats], M, LR, BETA, 5, COEFFS)
    W = [to_gpu(w.cpu().numpy()) for w in W]
    M = [to_gpu(x.cpu().numpy()) for x in M]
    for s in (1, 2):
        mu.muon_step(W, [to_gpu(m["grads"][s]) for m in mats], M, LR, BETA, 5, COEFFS)
    torch.cuda.synchronize()
    for a, b in zip(W + M, W1 + M1):
        assert torch.equal(a, b)


def test_error_paths_on_gpu():
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    w = torch.zeros((8, 8), device="cuda")
    g = torch.zeros((8, 8), device="cuda")
    m = torch.zeros((8, 8), device="cuda")
    with pytest.raises(mu.MuonError, match="EINVAL"):
        mu.muon_step([w], [g], [w], 0.02, 0.95, 5)  # momentum aliases params
    with pytest.raises(mu.MuonError, match="EINVAL"):
        mu.muon_step([w], [g], [m], float("nan"), 0.95, 5)
    with pytest.raises(mu.MuonError, match="EINVAL"):
        mu.muon_step([w], [g], [m], 0.02, 1.0, 5)
    with pytest.raises(mu.MuonError, match="EINVAL"):
        mu.muon_step([w], [g], [m], 0.02, 0.95, -1)
    mu.muon_step([], [], [], 0.02, 0.95, 5)  # n = 0 is a no-op


def test_injected_allocation_failure(monkeypatch):
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    mu.muon_release()
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    w = torch.zeros((8, 8), device="cuda")
    with pytest.raises(mu.MuonError, match="ENOMEM"):
        mu.muon_step([w], [torch.ones((8, 8), device="cuda")], [torch.zeros((8, 8), device="cuda")], 0.02, 0.95, 5)
    monkeypatch.delenv("MUON_TEST_FAIL_ALLOC")
    mu.muon_step([w], [torch.ones((8, 8), device="cuda")], [torch.zeros((8, 8), device="cuda")], 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert torch.isfinite(w).all()


def test_caller_workspace():
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(9)
    m = {"W": rng.standard_normal((200, 300)).astype(np.float32), "buf": np.zeros((200, 300), np.float32),
         "grads": [rng.standard_normal((200, 300)).astype(np.float32)]}
    need = mu.muon_workspace_bytes([(200, 300)])
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    mu.muon_set_workspace(base, need)
    try:
        Wg, Mg, Ug = gpu_step([m], "grads", 1)
        r = oracle_steps(m, 1)
        check_matrix("caller workspace", Wg[0], Mg[0], Ug[0], r, m["W"].astype(np.float64))
        with pytest.raises(mu.MuonError, match="ENOMEM"):
            gpu_step([{"W": np.zeros((512, 512), np.float32), "buf": np.zeros((512, 512), np.float32),
                       "grads": [np.ones((512, 512), np.float32)]}], "grads", 1)
    finally:
        mu.muon_set_workspace(None, 0)


@pytest.mark.parametrize("shape", [(64, 32, 3, 3), (300, 4, 5), (8, 3, 5, 5)])
def test_rank_above_two_is_the_flattened_matrix(shape):
    """A filter (out, in, kh, kw) is stepped as the out x (in kh kw) matrix:
    bit-identical to passing that 2-D view, and within the bar of the oracle."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(sum(shape))
    W0 = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    g = rng.standard_normal(shape).astype(np.float32)
    Wt, Gt, Mt = to_gpu(W0), to_gpu(g), torch.zeros(shape, device="cuda")
    Ut = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    mu.muon_step([Wt], [Gt], [Mt], LR, BETA, 5, COEFFS, updates=[Ut])
    m = mu.matrix_shape(shape)
    W2, G2, M2 = to_gpu(W0.reshape(m)), to_gpu(g.reshape(m)), torch.zeros(m, device="cuda")
    mu.muon_step([W2], [G2], [M2], LR, BETA, 5, COEFFS)
    torch.cuda.synchronize()
    assert torch.equal(Wt.reshape(m), W2) and torch.equal(Mt.reshape(m), M2)
    r = om.muon_step_tensor(W0, g, np.zeros_like(g), LR, BETA, 5, COEFFS)
    e = rel_f(bf16_to_np(Ut), r["O"])
    say(f"  {shape} as {m}: update relF {e:.2e}")
    assert bf16_to_np(Ut).shape == shape and e <= NS_TOL
