"""GPU parity of per-iteration coefficient schedules (one (a, b, c) triple per
Newton-Schulz iteration, triple k in iteration k): the HIP library against
the CPU oracle, same bars as the fixed-triple path."""
import numpy as np
import pytest

from gpu_helpers import (COEFFS, NS_TOL, bf16_gpu, bf16_to_np, check_matrix, empty_bf16, gpu_step, oracle_steps,
                         rel_f, say, torch_mod)
from oracle import muon_oracle as om
from optimizer_muon_step_amd import workloads as wl

pytestmark = pytest.mark.gpu

# Aggressive slope at zero first, then triples that settle towards 1 (the last
# one is the textbook quintic that converges to the polar factor).
SCHEDULE = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (2.0, -1.5, 0.5),
            (1.875, -1.25, 0.375)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import optimizer_muon_step_amd as mu
    mu._lib.load()
    yield
    torch.cuda.synchronize()


def test_schedule_step_c1():
    specs = wl.config_specs("c1")
    mats = [wl.make_matrix("c1", i, 2) for i in range(len(specs))]
    say(f"[schedule c1] {len(mats)} matrices, 2 steps")
    Wg, Mg, Ug = gpu_step(mats, "grads", 2, coeffs=SCHEDULE)
    for i, spec in enumerate(specs):
        r = oracle_steps(mats[i], 2, coeffs=SCHEDULE)
        check_matrix(f"c1[{i}] {spec.rows}x{spec.cols}", Wg[i], Mg[i], Ug[i], r, mats[i]["W"].astype(np.float64))


def test_schedule_ragged_shapes():
    rng = np.random.default_rng(21)
    shapes = [(1, 1), (129, 257), (257, 129), (5, 700), (384, 384)]
    mats = [{"W": rng.standard_normal(s).astype(np.float32), "buf": np.zeros(s, np.float32),
             "grads": [rng.standard_normal(s).astype(np.float32)]} for s in shapes]
    sched = SCHEDULE[:3]
    Wg, Mg, Ug = gpu_step(mats, "grads", 1, ns_steps=3, coeffs=sched)
    for i, (s, m) in enumerate(zip(shapes, mats)):
        r = oracle_steps(m, 1, ns_steps=3, coeffs=sched)
        check_matrix(f"{s}", Wg[i], Mg[i], Ug[i], r, m["W"].astype(np.float64))


def test_schedule_of_equal_triples_is_bit_identical_to_the_fixed_triple():
    torch = torch_mod()
    mats = [wl.make_matrix("c2", i, 1) for i in range(4)]
    W1, M1, U1 = gpu_step(mats, "grads", 1, coeffs=COEFFS)
    W2, M2, U2 = gpu_step(mats, "grads", 1, coeffs=[COEFFS] * 5)
    for a, b in zip(W1 + M1 + U1, W2 + M2 + U2):
        assert torch.equal(a, b)


def test_schedule_monomial_bit_exact():
    """One non-zero per row and column: every dot product has a single term,
    so each iteration's storage points must match the oracle bit for bit
    whatever triple the iteration uses."""
    rng = np.random.default_rng(22)
    n, m = 130, 260
    g = np.zeros((n, m), np.float32)
    cols = rng.permutation(m)[:n]
    g[np.arange(n), cols] = rng.integers(1, 8, n) * rng.choice([-1, 1], n)
    W = rng.standard_normal(g.shape).astype(np.float32)
    mat = {"W": W, "buf": np.zeros_like(W), "grads": [g]}
    Wg, Mg, Ug = gpu_step([mat], "grads", 1, coeffs=SCHEDULE)
    r = oracle_steps(mat, 1, coeffs=SCHEDULE)
    assert np.array_equal(bf16_to_np(Ug[0]), r["O"])
    assert np.array_equal(Wg[0].cpu().numpy(), r["W"])


@pytest.mark.parametrize("shape", [(256, 512), (300, 200), (64, 2304)])
def test_newton_schulz_schedule(shape):
    import optimizer_muon_step_amd as mu
    say(f"[ns schedule] shape={shape}")
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    x = rng.standard_normal(shape).astype(np.float32)
    x /= np.float32(np.linalg.norm(x.astype(np.float64)) + 1e-7)
    bits = om.bf16_bits(x)
    out = empty_bf16(shape)
    mu.muon_newton_schulz([bf16_gpu(bits)], [out], len(SCHEDULE), SCHEDULE)
    X0 = om.bf16_to_f32(bits)
    Xc, tr = om.canonical(X0)
    want = om.newton_schulz(np.ascontiguousarray(Xc), len(SCHEDULE), SCHEDULE)
    want = want.T if tr else want
    e = rel_f(bf16_to_np(out), want)
    say(f"  relF {e:.3e}")
    assert e <= NS_TOL
    # and the schedule really is applied in order: the reversed one differs
    rev = om.newton_schulz(np.ascontiguousarray(Xc), len(SCHEDULE), SCHEDULE[::-1])
    rev = rev.T if tr else rev
    assert rel_f(bf16_to_np(out), rev) > 10 * NS_TOL
