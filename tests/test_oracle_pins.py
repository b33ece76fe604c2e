"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test pins one part of the oracle to mathematics or to a hand-derived
value, chosen so that a plausible slip (a dropped term, a sign, a transposed
operand, a storage point in the wrong place, plain instead of Nesterov
momentum) fails at least one of them.  The mutation tests at the end plant
such slips in a copy of the oracle and check that the pins catch them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import muon_oracle as om
from exact_fp import bf16 as bf16_exact, fp32 as fp32_exact

COEFFS = om.DEFAULT_COEFFS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_f(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    d = np.linalg.norm(x - y)
    n = np.linalg.norm(y)
    return d / n if n > 0 else d


def p_scalar(sig, k, coeffs=COEFFS):
    """The quintic p(s) = a s + b s^3 + c s^5 applied k times to one number."""
    a, b, c = coeffs
    for _ in range(k):
        sig = a * sig + b * sig ** 3 + c * sig ** 5
    return sig


# ---------------------------------------------------------------- bfloat16 --

def _load_bf16_golden():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            src, dst = line.split()[:2]
            rows.append((int(src, 16), dst))
    return rows


def test_bf16_golden_bit_patterns():
    rows = _load_bf16_golden()
    assert len(rows) >= 20
    src = np.array([r[0] for r in rows], np.uint32).view(np.float32)
    got = oracle.bf16_bits(src)
    for (s, want), g in zip(rows, got):
        if want == "nan":
            assert (g & 0x7F80) == 0x7F80 and (g & 0x7F) != 0, f"{s:08X} -> {g:04X} is not NaN"
        else:
            assert int(g) == int(want, 16), f"{s:08X}: got {int(g):04X}, want {want}"


def test_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    # keep finite values, include many subnormals and exact ties
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]
    ties = (rng.integers(0, 2 ** 16, size=500, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    ties = ties[((ties >> 23) & 0xFF) != 0xFF]
    sub = rng.integers(0, 2 ** 23, size=500, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits, ties, sub]).view(np.float32)
    got = oracle.bf16_round(x)
    for xi, gi in zip(x.tolist(), got.tolist()):
        want = bf16_exact(xi)
        assert gi == want or (math.isinf(want) and math.isinf(gi) and (gi > 0) == (want > 0)), (xi, gi, want)


# ------------------------------------------------- singular-value closed form --

@pytest.mark.parametrize("shape", [(8, 12), (16, 16), (40, 24), (64, 96), (1, 7), (9, 1)])
@pytest.mark.parametrize("k", [1, 2, 5])
def test_exact_mode_equals_svd_closed_form(shape, k):
    """For X0 = U diag(s) V^T the iteration gives U diag(p^k(s)) V^T."""
    rng = np.random.default_rng(hash((shape, k)) % (2 ** 32))
    g = rng.standard_normal(shape)
    O, X0, s = om.orthogonalize(g, k, COEFFS, mode="exact")
    U, sig, Vt = np.linalg.svd(g * s, full_matrices=False)
    want = (U * p_scalar(sig, k)) @ Vt
    assert O.shape == g.shape
    assert rel_f(O, want) < 1e-8


def test_coefficient_triple_values():
    a, b, c = COEFFS
    # slope at zero of p is a; p(1) = a + b + c < 1: the aggressive, non-converging choice
    assert (a, b, c) == (3.4445, -4.7750, 2.0315)
    assert abs((a + b + c) - 0.701) < 1e-12
    assert abs(p_scalar(1.0, 5) - 0.696436) < 1e-6


def test_rank_one_gives_scaled_outer_product():
    """G = w u v^T has one singular value; after normalisation it is
    ||g|| / (||g|| + eps), and the output is p^5 of that times u v^T."""
    rng = np.random.default_rng(3)
    u = rng.standard_normal(24)
    v = rng.standard_normal(40)
    u /= np.linalg.norm(u)
    v /= np.linalg.norm(v)
    for w in (3.0, 1e-6):
        g = w * np.outer(u, v)
        O, _, _ = om.orthogonalize(g, 5, COEFFS, mode="exact")
        sig = w / (w + om.NORM_EPS)
        assert rel_f(O, p_scalar(sig, 5) * np.outer(u, v)) < 1e-10
    # the eps matters at w = 1e-6: sigma = 1/1.1 rather than 1
    assert abs(p_scalar(1e-6 / (1e-6 + 1e-7), 5) - p_scalar(1.0, 5)) > 1e-3


def test_one_by_one_and_diagonal_cases():
    for gval in (2.5, -0.75):
        O, _, _ = om.orthogonalize(np.array([[gval]]), 5, COEFFS, mode="exact")
        sig = abs(gval) / (abs(gval) + om.NORM_EPS)
        assert abs(O[0, 0] - math.copysign(p_scalar(sig, 5), gval)) < 1e-12
    O, _, _ = om.orthogonalize(np.diag([3.0, 4.0]), 5, COEFFS, mode="exact")
    n = 5.0 + om.NORM_EPS
    assert abs(O[0, 0] - p_scalar(3.0 / n, 5)) < 1e-12
    assert abs(O[1, 1] - p_scalar(4.0 / n, 5)) < 1e-12
    assert O[0, 1] == 0.0 and O[1, 0] == 0.0
    # hand-checked values: p^5(0.6) = 0.722876, p^5(0.8) = 1.119204
    assert abs(p_scalar(0.6, 5) - 0.722876) < 1e-6
    assert abs(p_scalar(0.8, 5) - 1.119204) < 1e-6


def test_orthogonal_input_maps_to_scaled_orthogonal():
    rng = np.random.default_rng(5)
    n = 32
    q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    O, _, _ = om.orthogonalize(q, 5, COEFFS, mode="exact")
    sig = math.sqrt(n) / (math.sqrt(n) + om.NORM_EPS) / math.sqrt(n)
    assert rel_f(O, p_scalar(sig, 5) * q) < 1e-10


# ----------------------------------------------- bf16 ("emul") mode pins --

def test_emul_singular_values_inside_band():
    """The bf16 iteration's output singular values lie where p^5 puts the
    input's (well-spread Gaussian, every normalised sigma above 3e-3):
    p^5 maps [3e-3, 1] into [0.6818, 1.2024]; allow a few bf16 ulps."""
    lo = min(p_scalar(s, 5) for s in np.linspace(3e-3, 1, 20001))
    hi = max(p_scalar(s, 5) for s in np.linspace(3e-3, 1, 20001))
    assert 0.68 < lo < 0.683 and 1.20 < hi < 1.21
    rng = np.random.default_rng(11)
    g = rng.standard_normal((128, 256)).astype(np.float32)
    O, X0, s = om.orthogonalize(g, 5, COEFFS, mode="emul")
    sv = np.linalg.svd(O.astype(np.float64), compute_uv=False)
    sv_in = np.linalg.svd(g.astype(np.float64) * float(s), compute_uv=False)
    assert sv_in.min() > 3e-3
    assert sv.min() > lo - 0.03 and sv.max() < hi + 0.03
    # and the emul result is close to the exact closed form of its own bf16 input
    O_ex = om.newton_schulz(X0.astype(np.float64), 5, COEFFS, mode="exact")
    assert rel_f(O, O_ex) < 3e-2


def test_emul_scale_invariance_power_of_two_bit_exact():
    rng = np.random.default_rng(12)
    g = rng.standard_normal((48, 80)).astype(np.float32)
    O1, _, _ = om.orthogonalize(g, 5, COEFFS)
    for j in (-3, 4):
        O2, _, _ = om.orthogonalize(g * np.float32(2.0 ** j), 5, COEFFS)
        assert np.array_equal(O1, O2)


def test_emul_transpose_equivariance():
    rng = np.random.default_rng(13)
    g = rng.standard_normal((40, 72)).astype(np.float32)
    O1, _, _ = om.orthogonalize(g, 5, COEFFS)
    O2, _, _ = om.orthogonalize(np.ascontiguousarray(g.T), 5, COEFFS)
    assert np.array_equal(O1.T, O2)  # canonicalisation makes this exact
    # square: no canonical transpose, so the two orders really differ; use a
    # well-conditioned matrix (a square Gaussian has singular values near 0,
    # which p^5 amplifies ~485x together with their rounding noise)
    q1, _ = np.linalg.qr(rng.standard_normal((48, 48)))
    q2, _ = np.linalg.qr(rng.standard_normal((48, 48)))
    sq = ((q1 * np.linspace(0.3, 1.0, 48)) @ q2.T).astype(np.float32)
    O3, _, _ = om.orthogonalize(sq, 5, COEFFS)
    O4, _, _ = om.orthogonalize(np.ascontiguousarray(sq.T), 5, COEFFS)
    # X^T X and X X^T round differently at every storage point; the two bf16
    # results agree only to the iteration's own noise level (~2e-2 measured)
    assert rel_f(O4, O3.T) < 5e-2
    O3e, _, _ = om.orthogonalize(sq, 5, COEFFS, mode="exact")
    O4e, _, _ = om.orthogonalize(np.ascontiguousarray(sq.T), 5, COEFFS, mode="exact")
    assert rel_f(O4e, O3e.T) < 1e-12


def test_emul_zero_rows_stay_zero():
    rng = np.random.default_rng(14)
    g = np.zeros((300, 48), np.float32)
    rows = rng.choice(300, 20, replace=False)
    g[rows] = rng.standard_normal((20, 48)).astype(np.float32)
    O, _, _ = om.orthogonalize(g, 5, COEFFS)
    mask = np.ones(300, bool)
    mask[rows] = False
    assert np.all(O[mask] == 0.0)
    assert np.all(np.abs(O[rows]).sum(axis=1) > 0)


def test_signed_permutation_equivariance():
    rng = np.random.default_rng(15)
    g = rng.standard_normal((24, 56))
    P = np.eye(24)[rng.permutation(24)] * rng.choice([-1.0, 1.0], 24)[:, None]
    Q = np.eye(56)[rng.permutation(56)] * rng.choice([-1.0, 1.0], 56)[None, :]
    Oe, _, _ = om.orthogonalize(g, 5, COEFFS, mode="exact")
    Oe2, _, _ = om.orthogonalize(P @ g @ Q, 5, COEFFS, mode="exact")
    assert rel_f(Oe2, P @ Oe @ Q) < 1e-12
    g32 = g.astype(np.float32)
    O, _, _ = om.orthogonalize(g32, 5, COEFFS)
    O2, _, _ = om.orthogonalize((P @ g32 @ Q).astype(np.float32), 5, COEFFS)
    assert rel_f(O2, P @ O @ Q) < 1e-2


def test_zero_matrix_leaves_params_unchanged():
    W = np.random.default_rng(16).standard_normal((16, 32)).astype(np.float32)
    z = np.zeros_like(W)
    r = om.muon_step_matrix(W, z, z, 0.02, 0.95, 5)
    assert np.all(r["O"] == 0.0)
    assert np.array_equal(r["W"], W)
    assert np.all(r["buf"] == 0.0)


# --------------------------------------------------------------- momentum --

def test_momentum_step_one_and_two():
    rng = np.random.default_rng(17)
    g1 = rng.standard_normal((20, 30)).astype(np.float32)
    g2 = rng.standard_normal((20, 30)).astype(np.float32)
    beta = 0.95
    z = np.zeros_like(g1)
    buf1, u1 = om.nesterov_momentum(g1, z, beta)
    assert np.array_equal(buf1, g1)  # from a zero buffer the buffer is the gradient
    buf2, u2 = om.nesterov_momentum(g2, buf1, beta)
    want_buf = beta * g1.astype(np.float64) + g2
    want_u = g2 + beta * want_buf  # Nesterov: look ahead on the updated buffer
    # two fp32 roundings each: error below 2^-23 of the terms' magnitudes
    mag_buf = beta * np.abs(g1.astype(np.float64)) + np.abs(g2)
    mag_u = np.abs(g2.astype(np.float64)) + beta * mag_buf
    assert np.all(np.abs(buf2 - want_buf) <= 2 ** -23 * mag_buf)
    assert np.all(np.abs(u2 - want_u) <= 2 ** -22 * mag_u)
    # the normalised, cast X0 of step 2 is the normalised Nesterov vector, to bf16 precision
    O, X0, s = om.orthogonalize(u2, 0, COEFFS)
    ref = want_u / np.linalg.norm(want_u)
    assert np.max(np.abs(O - ref)) <= 2 ** -8 * np.max(np.abs(ref)) + 1e-7
    # ... and is far from what plain heavy-ball momentum or plain SGD would give
    assert rel_f(O, want_buf / np.linalg.norm(want_buf)) > 0.05
    assert rel_f(O, g2 / np.linalg.norm(g2)) > 0.05


@pytest.mark.parametrize("mode,beta", [("exact", 0.9), ("exact", 0.95), ("emul", 0.5), ("emul", 0.75)])
def test_momentum_unrolled_sum_over_steps(mode, beta):
    """Readings R1 and R2 against their unrolled closed form: from a zero
    buffer, after k steps buf_k = sum_j beta^(k-j) g_j and the Nesterov vector
    is u_k = g_k + beta * buf_k.  Exact mode (fp64) must match the sum to
    rounding; in emul mode beta is a short binary fraction and the gradients
    small integers, so every intermediate is exact in fp32 and the sum must
    hold bit for bit.  A look-ahead on the old buffer (u = g + beta * buf_{k-1})
    or an EMA buffer (beta * buf + (1 - beta) g) fails both."""
    rng = np.random.default_rng(23)
    k_steps = 4
    if mode == "exact":
        gs = [rng.standard_normal((9, 13)) for _ in range(k_steps)]
    else:
        gs = [rng.integers(-8, 9, size=(9, 13)).astype(np.float32) for _ in range(k_steps)]
    buf = np.zeros_like(gs[0])
    for k in range(1, k_steps + 1):
        buf, u = om.nesterov_momentum(gs[k - 1], buf, beta, mode)
        want_buf = sum(beta ** (k - j) * np.asarray(gs[j - 1], np.float64) for j in range(1, k + 1))
        want_u = np.asarray(gs[k - 1], np.float64) + beta * want_buf
        if mode == "exact":
            assert buf.dtype == np.float64 and u.dtype == np.float64
            assert np.max(np.abs(buf - want_buf)) <= 1e-13 * np.max(np.abs(want_buf))
            assert np.max(np.abs(u - want_u)) <= 1e-13 * np.max(np.abs(want_u))
        else:
            assert buf.dtype == np.float32 and u.dtype == np.float32
            assert np.array_equal(buf.astype(np.float64), want_buf)
            assert np.array_equal(u.astype(np.float64), want_u)
        if k >= 2:
            old = want_buf - np.asarray(gs[k - 1], np.float64)  # beta * buf_{k-1}
            assert np.max(np.abs(u - (np.asarray(gs[k - 1], np.float64) + old))) > 0.1


def test_frobenius_scale_eps_reading():
    u = np.array([[3e-7, 4e-7]], np.float32)
    s = om.frobenius_scale(u)
    norm = math.sqrt(float(np.float32(3e-7)) ** 2 + float(np.float32(4e-7)) ** 2)
    assert s == np.float32(1.0 / (norm + 1e-7))
    assert abs(float(s) * 6e-7 - 1.0) < 1e-6


# ------------------------------------------------------- monomial inputs --

def _monomial(n, m, rng, transpose=False):
    """One non-zero per row and column (n <= m), small integers: every dot
    product of the iteration has a single non-zero term, so the result does
    not depend on summation order and can be derived entry by entry."""
    g = np.zeros((n, m), np.float32)
    cols = rng.permutation(m)[:n]
    vals = rng.integers(1, 8, n) * rng.choice([-1, 1], n)
    g[np.arange(n), cols] = vals
    return (g.T.copy(), cols, vals) if transpose else (g, cols, vals)


def _scalar_chain(vals, ss, beta, lr, w0, coeffs, k):
    """Entry-by-entry derivation with exact rational rounding at each
    storage point (fresh momentum: buf = g, u = g + beta*g)."""
    a, b, c = (fp32_exact(v) for v in coeffs)
    fb = fp32_exact(beta)
    s = fp32_exact(1.0 / (math.sqrt(ss) + 1e-7))
    out = []
    for v, w in zip(vals, w0):
        v = float(v)
        u = fp32_exact(v + fp32_exact(fb * v))
        x = bf16_exact(fp32_exact(u * s))
        for _ in range(k):
            A = bf16_exact(fp32_exact(x * x))
            B = bf16_exact(fp32_exact(fp32_exact(b * A) + fp32_exact(c * fp32_exact(A * A))))
            x = bf16_exact(fp32_exact(fp32_exact(a * x) + fp32_exact(B * x)))
        out.append((x, fp32_exact(w - fp32_exact(fp32_exact(lr) * x))))
    return out


@pytest.mark.parametrize("shape,transpose", [((12, 20), False), ((16, 16), False), ((10, 26), True)])
def test_monomial_inputs_bit_exact(shape, transpose):
    rng = np.random.default_rng(shape[0] * 100 + shape[1])
    g, cols, vals = _monomial(*shape, rng, transpose)
    W = rng.standard_normal(g.shape).astype(np.float32)
    beta, lr = 0.95, 0.02
    r = om.muon_step_matrix(W, g, np.zeros_like(g), lr, beta, 5)
    u = r["u"].astype(np.float64)
    ss = float(np.sum(u * u))
    rows = np.arange(shape[0])
    if transpose:
        w0 = W[cols, rows]
    else:
        w0 = W[rows, cols]
    chain = _scalar_chain(vals, ss, beta, lr, w0, om.DEFAULT_COEFFS, 5)
    O = r["O"]
    for i, (x, w) in enumerate(chain):
        rr, cc = (cols[i], i) if transpose else (i, cols[i])
        assert O[rr, cc] == x, (i, O[rr, cc], x)
        assert r["W"][rr, cc] == w
    mask = np.ones(g.shape, bool)
    if transpose:
        mask[cols, rows] = False
    else:
        mask[rows, cols] = False
    assert np.all(O[mask] == 0.0)
    assert np.array_equal(r["W"][mask], W[mask])


# ------------------------------------------------ brute force, tiny sizes --

def _bf_matmul(X, Y):
    """Triple loop, sequential fp32 accumulation, exact rational rounding."""
    n, k = len(X), len(X[0])
    m = len(Y[0])
    out = [[0.0] * m for _ in range(n)]
    for i in range(n):
        for j in range(m):
            acc = 0.0
            for t in range(k):
                acc = fp32_exact(acc + fp32_exact(X[i][t] * Y[t][j]))
            out[i][j] = acc
    return out


def _brute_force_orthogonalize(g, k, coeffs, beta):
    a, b, c = (fp32_exact(v) for v in coeffs)
    fb = fp32_exact(beta)
    rows, cols = g.shape
    u = [[fp32_exact(float(v) + fp32_exact(fb * float(v))) for v in row] for row in g]
    ss = sum(v * v for row in u for v in row)
    s = fp32_exact(1.0 / (math.sqrt(ss) + 1e-7))
    if rows > cols:
        u = [list(r) for r in zip(*u)]
    X = [[bf16_exact(fp32_exact(v * s)) for v in row] for row in u]
    for _ in range(k):
        Xt = [list(r) for r in zip(*X)]
        A = [[bf16_exact(v) for v in row] for row in _bf_matmul(X, Xt)]
        AA = _bf_matmul(A, A)
        B = [[bf16_exact(fp32_exact(fp32_exact(b * A[i][j]) + fp32_exact(c * AA[i][j])))
              for j in range(len(A))] for i in range(len(A))]
        BX = _bf_matmul(B, X)
        X = [[bf16_exact(fp32_exact(fp32_exact(a * X[i][j]) + BX[i][j]))
              for j in range(len(X[0]))] for i in range(len(X))]
    if rows > cols:
        X = [list(r) for r in zip(*X)]
    return np.array(X)


@pytest.mark.parametrize("shape", [(6, 10), (8, 8), (11, 5)])
def test_brute_force_tiny(shape):
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    g = rng.standard_normal(shape).astype(np.float32)
    beta = 0.95
    want = _brute_force_orthogonalize(g, 5, COEFFS, beta)
    _, u = om.nesterov_momentum(g, np.zeros_like(g), beta)
    got, _, _ = om.orthogonalize(u, 5, COEFFS)
    assert rel_f(got, want) < 2e-3


# ------------------------------------------------------------- mutations --

def _svd_pin_holds(orth):
    rng = np.random.default_rng(99)
    for shape in ((12, 20), (16, 16)):
        g = rng.standard_normal(shape)
        try:
            O = orth(g)
        except ValueError:
            return False
        U, sig, Vt = np.linalg.svd(g / (np.linalg.norm(g) + om.NORM_EPS), full_matrices=False)
        if not rel_f(O, (U * p_scalar(sig, 5)) @ Vt) < 1e-8:
            return False
    return True


def test_mutations_are_caught(monkeypatch):
    """Plant plausible slips in the oracle and check the pins reject them."""
    good = lambda g: om.orthogonalize(g, 5, COEFFS, mode="exact")[0]
    assert _svd_pin_holds(good)

    def dropped_c(X, a, b, c, mode="emul"):
        X = np.asarray(X, np.float64)
        A = X @ X.T
        return a * X + (b * A) @ X

    def wrong_sign(X, a, b, c, mode="emul"):
        X = np.asarray(X, np.float64)
        A = X @ X.T
        return a * X - (b * A + c * A @ A) @ X

    def transposed_gram(X, a, b, c, mode="emul"):
        X = np.asarray(X, np.float64)
        A = X @ X  # X X instead of X X^T
        return a * X + (b * A + c * A @ A) @ X

    def swapped_coeffs(X, a, b, c, mode="emul"):
        X = np.asarray(X, np.float64)
        A = X @ X.T
        return a * X + (c * A + b * A @ A) @ X

    for bad in (dropped_c, wrong_sign, transposed_gram, swapped_coeffs):
        monkeypatch.setattr(om, "ns_iteration", bad)
        assert not _svd_pin_holds(good), bad.__name__
    monkeypatch.undo()

    # plain momentum instead of Nesterov changes X0 of step 2
    def heavy_ball(g, buf, beta, mode="emul"):
        g = np.asarray(g, np.float32)
        b = (np.float32(beta) * np.asarray(buf, np.float32)) + g
        return b, b

    rng = np.random.default_rng(18)
    g1 = rng.standard_normal((20, 30)).astype(np.float32)
    g2 = rng.standard_normal((20, 30)).astype(np.float32)
    monkeypatch.setattr(om, "nesterov_momentum", heavy_ball)
    buf1, _ = om.nesterov_momentum(g1, np.zeros_like(g1), 0.95)
    _, u2 = om.nesterov_momentum(g2, buf1, 0.95)
    want_u = g2 + 0.95 * (0.95 * g1.astype(np.float64) + g2)
    assert np.max(np.abs(u2 - want_u) / (np.abs(want_u) + 1e-30)) > 1e-3
    monkeypatch.undo()

    # a storage point moved (B kept in fp32) breaks the monomial bit-exactness
    def b_not_rounded(X, a, b, c, mode="emul"):
        X = np.asarray(X, np.float32)
        A = om.bf16_round(X @ X.T)
        B = (np.float32(b) * A) + (np.float32(c) * (A @ A))
        return om.bf16_round((np.float32(a) * X) + B @ X)

    monkeypatch.setattr(om, "ns_iteration", b_not_rounded)
    with pytest.raises(AssertionError):
        test_monomial_inputs_bit_exact((12, 20), False)


# ------------------------------------------------- coefficient schedules --
# One (a, b, c) per iteration.  In exact arithmetic the iteration still acts
# on each singular value separately, now through the composition of the
# per-iteration polynomials, in iteration order.

SCHEDULE = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (2.0, -1.5, 0.5),
            (1.875, -1.25, 0.375)]


def p_composed(sig, schedule):
    for coeffs in schedule:
        sig = p_scalar(sig, 1, coeffs)
    return sig


@pytest.mark.parametrize("shape", [(12, 20), (16, 16), (24, 40)])
def test_schedule_singular_value_closed_form(shape):
    rng = np.random.default_rng(41)
    g = rng.standard_normal(shape)
    O = om.orthogonalize(g, len(SCHEDULE), SCHEDULE, mode="exact")[0]
    U, sig, Vt = np.linalg.svd(g / (np.linalg.norm(g) + om.NORM_EPS), full_matrices=False)
    assert rel_f(O, (U * p_composed(sig, SCHEDULE)) @ Vt) < 1e-8


def test_schedule_order_matters():
    """The reversed schedule is a different map: a slip that applied the
    triples in the wrong order would fail the closed form above."""
    rng = np.random.default_rng(42)
    g = rng.standard_normal((12, 20))
    fwd = om.orthogonalize(g, len(SCHEDULE), SCHEDULE, mode="exact")[0]
    rev = om.orthogonalize(g, len(SCHEDULE), SCHEDULE[::-1], mode="exact")[0]
    assert rel_f(fwd, rev) > 1e-3


def test_schedule_of_equal_triples_is_the_fixed_triple():
    """emul mode, bit for bit: a schedule repeating the default triple is the
    default iteration."""
    rng = np.random.default_rng(43)
    X0 = om.bf16_round(rng.standard_normal((20, 36)).astype(np.float32) * np.float32(0.05))
    a = om.newton_schulz(X0, 4, COEFFS)
    b = om.newton_schulz(X0, 4, [COEFFS] * 4)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_schedule_rank_one_scalar_chain():
    """Rank 1 (normalised sigma = 1 up to eps): O = f(1) u v^T with f the
    composed polynomial, computed by hand here."""
    rng = np.random.default_rng(44)
    u = rng.standard_normal(9)
    v = rng.standard_normal(15)
    g = np.outer(u, v)
    O = om.orthogonalize(g, len(SCHEDULE), SCHEDULE, mode="exact")[0]
    sigma = np.linalg.norm(g) / (np.linalg.norm(g) + om.NORM_EPS)
    s = sigma
    for a, b, c in SCHEDULE:
        s = a * s + b * s ** 3 + c * s ** 5
    want = s * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert rel_f(O, want) < 1e-12


def test_textbook_quintic_schedule_reaches_the_polar_factor():
    """With every triple (15/8, -10/8, 3/8), the textbook quintic
    Newton-Schulz polar iteration (p(1) = 1, p'(1) = p''(1) = 0), the
    iterate converges to U V^T, the orthogonal polar factor of the input."""
    rng = np.random.default_rng(45)
    Q1, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    Q2, _ = np.linalg.qr(rng.standard_normal((16, 10)))
    sig = np.linspace(0.2, 1.0, 10)          # condition number 5
    g = (Q1 * sig) @ Q2.T                      # 10 x 16
    O = om.orthogonalize(g, 20, [(1.875, -1.25, 0.375)] * 20, mode="exact")[0]
    U, _, Vt = np.linalg.svd(g, full_matrices=False)
    assert rel_f(O, U @ Vt) < 1e-12


def test_schedule_shape_is_checked():
    with pytest.raises(ValueError):
        om.newton_schulz(np.zeros((4, 6), np.float32), 3, [COEFFS] * 2)


# ------------------------------------------------------------ rank > 2 --

def test_rank_four_filter_is_its_im2col_matrix():
    """Reading R10: a conv filter (out, in, kh, kw) is orthogonalised as the
    matrix whose row o holds, in order over (in, y, x), the filter taps; that
    matrix is built here tap by tap, and the exact-mode result must be its
    SVD closed form, folded back the same way."""
    rng = np.random.default_rng(60)
    o, i, kh, kw = 6, 4, 3, 3
    g = rng.standard_normal((o, i, kh, kw))
    M = np.zeros((o, i * kh * kw))
    for a in range(o):
        col = 0
        for b in range(i):
            for y in range(kh):
                for x in range(kw):
                    M[a, col] = g[a, b, y, x]
                    col += 1
    r = om.muon_step_tensor(np.zeros_like(g), g, np.zeros_like(g), 1.0, 0.0, 5, COEFFS, mode="exact")
    U, sig, Vt = np.linalg.svd(M / (np.linalg.norm(M) + om.NORM_EPS), full_matrices=False)
    want = (U * p_scalar(sig, 5)) @ Vt
    got = np.zeros_like(want)
    for a in range(o):
        col = 0
        for b in range(i):
            for y in range(kh):
                for x in range(kw):
                    got[a, col] = r["O"][a, b, y, x]
                    col += 1
    assert r["O"].shape == g.shape
    assert rel_f(got, want) < 1e-8
    # W <- W - lr O in the tensor's own shape
    assert np.allclose(r["W"], -r["O"], atol=0)


def test_rank_three_tall_tensor_is_transposed_like_a_tall_matrix():
    """(12, 2, 3) is the 12 x 6 matrix: more rows than columns, so it is
    iterated transposed; emul mode must equal the 2-D call bit for bit."""
    rng = np.random.default_rng(61)
    g = rng.standard_normal((12, 2, 3)).astype(np.float32)
    W = rng.standard_normal((12, 2, 3)).astype(np.float32)
    r3 = om.muon_step_tensor(W, g, np.zeros_like(g), 0.02, 0.95, 5)
    r2 = om.muon_step_matrix(W.reshape(12, 6), g.reshape(12, 6), np.zeros((12, 6), np.float32), 0.02, 0.95, 5)
    assert np.array_equal(r3["O"].reshape(12, 6), r2["O"]) and np.array_equal(r3["W"].reshape(12, 6), r2["W"])
    with pytest.raises(ValueError):
        om.muon_step_tensor(W[0, 0], g[0, 0], g[0, 0], 0.02, 0.95, 5)
