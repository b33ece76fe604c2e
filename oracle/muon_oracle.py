"""Plain CPU oracle of one Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference the HIP library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path never calls it and shares no code with it.

What it computes, for each 2-D parameter matrix independently (sources are
the web pages the method is described on):

  * "New optimizer" thread by Keller Jordan (xunroll.com/thread/1842300916864844014),
    tweet 2/8: the update is SGD-Nesterov momentum, orthogonalised.
    Tweet 5/8: orthogonalise each parameter's update *after* applying Nesterov
    momentum, with a quintic Newton-Schulz iteration, run in bfloat16.
    Tweet 6/8: the quintic coefficients are chosen to maximise the slope at 0,
    accepting that the iteration does not converge exactly.
  * "07. Training neural networks" (llm-generalization-bounds explainer),
    section "Momentum": PyTorch's SGD keeps the running sum u = beta*u + g
    without a (1 - beta) factor, which only rescales the learning rate.

Readings taken where the pages are silent (each one is a choice, not a quote):

  R1 momentum buffer      buf <- beta*buf + g           (PyTorch SGD convention)
  R2 Nesterov look-ahead  u   <- g + beta*buf           (on the updated buffer)
  R3 normalisation        s = 1 / (||u||_F + 1e-7), sum of squares in fp64,
                          s rounded once to fp32
  R4 orientation          a matrix with more rows than columns is transposed so
                          the iteration always sees m <= n; the update is
                          transposed back
  R5 storage points       X0, A = X X^T, B = b A + c A A and every new X are
                          stored in bfloat16 (round-to-nearest-even); every
                          product accumulates in fp32 from bf16 operands; the
                          epilogue combinations are done in fp32 with one
                          rounding per operation and no fused multiply-add
  R6 coefficients         one (a, b, c) triple for every iteration, default
                          (3.4445, -4.7750, 2.0315); these values are not
                          printed on the pages.  Or a schedule: one triple per
                          iteration, triple k used in iteration k (tweet 6/8
                          presents the coefficients as a trade-off between
                          slope at zero and closeness to 1; choosing them per
                          iteration is the plain extension of that choice)
  R7 apply                W <- W - lr * O with no extra scale and no weight
                          decay (the thread's replies report weight decay as
                          worse), rounded once per operation in fp32
  R10 rank > 2            a parameter of shape (d0, d1, ..., dk) is the matrix
                          d0 x (d1 ... dk), its trailing dimensions flattened
                          in row-major order: the im2col view of a
                          convolution filter that a reply to the thread
                          suggests for tensors of any shape

Two modes:
  "emul"  fp32 arithmetic with bf16 rounding at the R5 storage points (parity)
  "exact" fp64 everywhere, no bf16 (pins the algebra against closed forms)
"""

from __future__ import annotations

import numpy as np

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
NORM_EPS = 1e-7

# ----------------------------------------------------------------------------
# bfloat16 round-to-nearest-even, emulated on fp32 bit patterns.
# bfloat16 is the upper half of an IEEE binary32 word (1 sign, 8 exponent,
# 7 fraction bits).  Rounding adds 0x7FFF plus the lowest kept bit, so exact
# halves go to the even neighbour; NaNs are kept NaN (forced quiet).
# ----------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """fp32 values -> uint16 bfloat16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    hi = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(x)
    hi = np.where(nan, (bits >> np.uint64(16)).astype(np.uint32) | np.uint32(0x0040), hi)
    return (hi & np.uint32(0xFFFF)).astype(np.uint16)


def bf16_to_f32(h) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> fp32 values (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------
# Step pieces.  Each takes and returns plain numpy arrays.
# ----------------------------------------------------------------------------


def nesterov_momentum(g, buf, beta, mode="emul"):
    """Readings R1 and R2: buf <- beta*buf + g, then u <- g + beta*buf.

    In "emul" mode every operation is one fp32 rounding (numpy does not fuse
    the multiply into the add)."""
    if mode == "exact":
        g = np.asarray(g, np.float64)
        buf_new = beta * np.asarray(buf, np.float64) + g
        return buf_new, g + beta * buf_new
    g = np.asarray(g, np.float32)
    b = np.float32(beta)
    buf_new = (b * np.asarray(buf, np.float32)) + g
    u = g + (b * buf_new)
    return buf_new.astype(np.float32), u.astype(np.float32)


def frobenius_scale(u, mode="emul"):
    """Reading R3: s = 1 / (||u||_F + 1e-7).  The sum of squares is taken in
    fp64 (every fp32 square is exact there); s is rounded to fp32 once."""
    ss = float(np.sum(np.square(np.asarray(u, np.float64))))
    s = 1.0 / (np.sqrt(ss) + NORM_EPS)
    return s if mode == "exact" else np.float32(s)


def canonical(u):
    """Reading R4: present the matrix with m <= n rows.  Returns (view, transposed)."""
    rows, cols = u.shape
    if rows > cols:
        return u.T, True
    return u, False


def ns_iteration(X, a, b, c, mode="emul"):
    """One quintic Newton-Schulz iteration X <- a X + (b A + c A A) X, A = X X^T.

    "emul" follows reading R5: A and B and the new X are rounded to bf16;
    the three products accumulate in fp32 (BLAS sgemm on bf16-valued fp32
    operands, whose products are exact in fp32)."""
    if mode == "exact":
        X = np.asarray(X, np.float64)
        A = X @ X.T
        B = b * A + c * (A @ A)
        return a * X + B @ X
    X = np.asarray(X, np.float32)
    fa, fb, fc = np.float32(a), np.float32(b), np.float32(c)
    A = bf16_round(X @ X.T)
    AA = A @ A
    B = bf16_round((fb * A) + (fc * AA))
    BX = B @ X
    return bf16_round((fa * X) + BX)


def coefficient_schedule(coeffs, ns_steps):
    """Reading R6: the (a, b, c) used in each iteration.  `coeffs` is one
    triple (used every time) or ns_steps triples (triple k in iteration k)."""
    arr = np.asarray(coeffs, dtype=np.float64)
    if arr.shape == (3,):
        return [tuple(float(v) for v in arr)] * ns_steps
    if arr.shape == (ns_steps, 3):
        return [tuple(float(v) for v in row) for row in arr]
    raise ValueError(f"coeffs must be one triple or {ns_steps} triples, got shape {arr.shape}")


def newton_schulz(X0, ns_steps, coeffs=DEFAULT_COEFFS, mode="emul"):
    """ns_steps iterations on a canonical (m <= n) matrix; returns the final X."""
    X = X0
    for a, b, c in coefficient_schedule(coeffs, ns_steps):
        X = ns_iteration(X, a, b, c, mode)
    return X


def orthogonalize(u, ns_steps, coeffs=DEFAULT_COEFFS, mode="emul"):
    """Normalise, canonicalise, cast to bf16 ("emul") and iterate.
    Returns (O in the caller's orientation, X0 canonical, s)."""
    s = frobenius_scale(u, mode)
    uc, transposed = canonical(u)
    if mode == "exact":
        X0 = np.asarray(uc, np.float64) * s
    else:
        X0 = bf16_round(np.asarray(uc, np.float32) * s)
    X = newton_schulz(X0, ns_steps, coeffs, mode)
    O = X.T if transposed else X
    return np.ascontiguousarray(O), X0, s


def apply_update(W, O, lr, mode="emul"):
    """Reading R7: W <- W - lr * O (fp32 product, then fp32 difference)."""
    if mode == "exact":
        return np.asarray(W, np.float64) - lr * np.asarray(O, np.float64)
    return (np.asarray(W, np.float32) - (np.float32(lr) * np.asarray(O, np.float32))).astype(np.float32)


def muon_step_matrix(W, g, buf, lr, beta, ns_steps, coeffs=DEFAULT_COEFFS, mode="emul"):
    """One Muon step on one matrix.  Returns a dict with the new W and buf,
    the update O (caller orientation), X0 (canonical) and the scale s."""
    buf_new, u = nesterov_momentum(g, buf, beta, mode)
    O, X0, s = orthogonalize(u, ns_steps, coeffs, mode)
    W_new = apply_update(W, O, lr, mode)
    return {"W": W_new, "buf": buf_new, "O": O, "X0": X0, "s": s, "u": u}


def muon_step_tensor(W, g, buf, lr, beta, ns_steps, coeffs=DEFAULT_COEFFS, mode="emul"):
    """Reading R10: one Muon step on a parameter of rank >= 2, taken as the
    matrix (first dimension) x (product of the others).  Results come back in
    the tensor's shape."""
    shape = np.shape(W)
    if len(shape) < 2:
        raise ValueError("rank >= 2 expected")
    m = (shape[0], int(np.prod(shape[1:])))
    r = muon_step_matrix(np.reshape(W, m), np.reshape(g, m), np.reshape(buf, m), lr, beta, ns_steps, coeffs, mode)
    return {k: (np.reshape(v, shape) if k in ("W", "buf", "O", "u") else v) for k, v in r.items()}
