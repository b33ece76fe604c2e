"""Large sizes: one 16384 x 65536 step (and its transpose).  The bf16 iterate
alone is 2 GiB and every fp32 array 4 GiB, so element and byte offsets run
far past 2^31 bytes in every kernel.  The gradient is monomial (one non-zero
per row and at most one per column, small integers): every dot product of
the Newton-Schulz iteration then has a single term, each non-zero evolves on
its own, and the oracle's emulated iteration on the diagonal matrix of the
distinct normalised values gives each result.  The GPU must match those bit
for bit, and every other element must stay exactly zero."""
import numpy as np
import pytest

from gpu_helpers import BETA, COEFFS, LR, say, torch_mod
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
    mu.muon_release()
    torch.cuda.empty_cache()


def _expected(vals):
    """Oracle values at the non-zeros: momentum, update O and new W (from
    W = 0), element for element."""
    buf, u = om.nesterov_momentum(vals, np.zeros_like(vals), BETA)
    s = om.frobenius_scale(u)  # the zeros add nothing to the norm
    x0 = om.bf16_round(u * s)
    distinct, inverse = np.unique(x0, return_inverse=True)
    o_distinct = np.diag(om.newton_schulz(np.diag(distinct), 5, COEFFS))
    o = o_distinct[inverse].astype(np.float32)
    w = om.apply_update(np.zeros_like(o), o, LR)
    return buf, o, w


@pytest.mark.parametrize("transpose", [False, True])
def test_largest_monomial_step_bit_exact(transpose):
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    m, n = 16384, 65536
    shape = (n, m) if transpose else (m, n)
    say(f"[large monomial] shape={shape}")
    rng = np.random.default_rng(77 + transpose)
    cols = rng.permutation(n)[:m].astype(np.int64)
    vals = (rng.integers(1, 8, m) * rng.choice([-1, 1], m)).astype(np.float32)
    ri, ci = (cols, np.arange(m)) if transpose else (np.arange(m), cols)
    ri_t, ci_t = torch.from_numpy(ri).cuda(), torch.from_numpy(ci).cuda()
    G = torch.zeros(shape, device="cuda")
    G[ri_t, ci_t] = torch.from_numpy(vals).cuda()
    W = torch.zeros_like(G)
    M = torch.zeros_like(G)
    U = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    mu.muon_step([W], [G], [M], LR, BETA, 5, COEFFS, updates=[U])
    torch.cuda.synchronize()
    buf, o, w = _expected(vals)
    got_m = M[ri_t, ci_t].cpu().numpy()
    got_o = U[ri_t, ci_t].float().cpu().numpy()
    got_w = W[ri_t, ci_t].cpu().numpy()
    say(f"  non-zeros: M {int(torch.count_nonzero(M))}, O {int(torch.count_nonzero(U))}, "
        f"W {int(torch.count_nonzero(W))} of {m}; |O| in [{np.abs(o).min():.4f}, {np.abs(o).max():.4f}]")
    assert np.array_equal(got_m, buf)
    assert np.array_equal(got_o, o)
    assert np.array_equal(got_w, w)
    assert np.count_nonzero(o) == m and np.count_nonzero(w) == m
    for t in (M, U, W):
        assert int(torch.count_nonzero(t)) == m  # every other element exactly zero
    del G, W, M, U
    torch.cuda.empty_cache()
