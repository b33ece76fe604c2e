"""Plain CPU oracle of one multi-tensor AdamW step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference the HIP library's AdamW entry point is checked against.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path never calls it and shares no code with it.

What it computes, for every parameter tensor independently (elementwise):
the "07. Training neural networks" page (llm-generalization-bounds explainer),
section "Adam, weight decay and AdamW" and its derivation block "Adam's bias
correction and AdamW's decoupling, derived":

    theta <- (1 - lr * lambda) * theta           decoupled weight decay, first
    u     <- beta1 * u + (1 - beta1) * g         running mean of gradients
    v     <- beta2 * v + (1 - beta2) * g * g     running mean of squared gradients
    uhat  =  u / (1 - beta1^t),  vhat = v / (1 - beta2^t)     bias corrections
    theta <- theta - lr * uhat / (sqrt(vhat) + eps)

with u = v = 0 before the first step and t = 1 on the first step.  The
thread's replies route every parameter that is not a hidden 2-D matrix to
AdamW; the GPT-2 lecture pages apply weight decay to matrices and not to 1-D
parameters, and fuse the AdamW update over all tensors.

Readings taken where the pages are silent (each is a choice, not a quote):

  W1 order            the decay multiplies theta before the Adam step, and
                      the moments see the loss gradient alone (decoupled)
  W2 step count       t is supplied by the caller, >= 1, one value for every
                      tensor of a call
  W3 precision        fp32 storage and arithmetic, one rounding per
                      operation in the order written above, no fused
                      multiply-add; division and square root correctly
                      rounded.  Scalars per call: lr, beta1, beta2, eps and
                      each lambda are fp32 values; 1 - beta1, 1 - beta2,
                      1 - beta1^t and 1 - beta2^t are evaluated in fp64 from
                      those fp32 values and rounded once to fp32; the decay
                      factor is fp32(1 - fp32(lr * lambda)), per tensor
  W4 expression form  (1 - beta2) * g * g is ((1 - beta2) * g) * g, and
                      lr * uhat / (...) is (lr * uhat) / (...), as written

Two modes:
  "emul"   fp32 with the W3 rounding (parity with the GPU, bit for bit)
  "exact"  fp64 everywhere (pins the algebra against the pages' printed
           worked example and closed forms)
"""

from __future__ import annotations

import numpy as np

DEFAULT_BETAS = (0.9, 0.999)
DEFAULT_EPS = 1e-8


def call_constants(lr, beta1, beta2, eps, weight_decay, step, mode="emul"):
    """The per-call scalars of one step in the mode's float type (reading W3).

    emul: lr, the betas, eps and lambda are fp32 values; 1 - beta_k and the
    bias-correction denominators 1 - beta_k^t are evaluated in fp64 from
    those fp32 values and rounded once to fp32; the decay factor is
    fp32(1 - fp32(lr * lambda)).  exact: the same quantities in fp64 from the
    arguments as given."""
    t = int(step)
    if t < 1:
        raise ValueError("step counts from 1")
    T = np.float64 if mode == "exact" else np.float32
    lr_t, b1, b2, eps_t, lam = (T(x) for x in (lr, beta1, beta2, eps, weight_decay))
    return {
        "T": T, "lr": lr_t, "beta1": b1, "beta2": b2, "eps": eps_t,
        "omb1": T(1.0 - float(b1)), "omb2": T(1.0 - float(b2)),
        "bc1": T(1.0 - float(b1) ** t), "bc2": T(1.0 - float(b2) ** t),
        "decay": T(1.0) - (lr_t * lam),
    }


def adamw_step(p, g, u, v, lr, beta1=DEFAULT_BETAS[0], beta2=DEFAULT_BETAS[1], eps=DEFAULT_EPS,
               weight_decay=0.0, step=1, mode="emul"):
    """One AdamW step on one tensor.  Returns (p_new, u_new, v_new).

    Both modes run the same sequence in the mode's float type: the decoupled
    decay scales theta (W1); the two running means absorb g and g*g; theta
    then moves against the bias-corrected first mean over the square root of
    the bias-corrected second mean plus eps.  In emul mode every numpy
    operation below is one fp32 rounding, in the W4 expression forms."""
    k = call_constants(lr, beta1, beta2, eps, weight_decay, step, mode)
    T = k["T"]
    p, g, u, v = (np.asarray(x, T) for x in (p, g, u, v))
    p_decayed = p * k["decay"]
    mean = (k["beta1"] * u) + (k["omb1"] * g)
    mean_sq = (k["beta2"] * v) + ((k["omb2"] * g) * g)
    move = (k["lr"] * (mean / k["bc1"])) / (np.sqrt(mean_sq / k["bc2"]) + k["eps"])
    return p_decayed - move, mean, mean_sq


def adamw_multi(params, grads, exp_avg, exp_avg_sq, lr, beta1=DEFAULT_BETAS[0], beta2=DEFAULT_BETAS[1],
                eps=DEFAULT_EPS, weight_decay=0.0, step=1, mode="emul"):
    """One step over a list of tensors; weight_decay is one value or one per
    tensor.  Returns a list of (p, u, v)."""
    n = len(params)
    wds = list(weight_decay) if np.ndim(weight_decay) else [weight_decay] * n
    return [adamw_step(params[i], grads[i], exp_avg[i], exp_avg_sq[i], lr, beta1, beta2, eps, wds[i], step, mode)
            for i in range(n)]


def untie_state(p, u, v, transpose=False):
    """Delayed untying (the "nanoGPT Speedrun Techniques: How Delayed Untying
    Solves the Sparse Gradient Problem" page, section "Option B: Delayed
    Untying"): the new parameter starts as a copy of the shared one together
    with both AdamW moments, so that its trajectory continues from the shared
    point.  With `transpose` the copies are laid out as the transpose (the
    output layer stored d_model x vocab, the page's description of lm_head
    against the vocab x d_model embedding)."""
    f = (lambda a: np.ascontiguousarray(np.asarray(a).T)) if transpose else (lambda a: np.array(a, copy=True))
    return f(p), f(u), f(v)
