"""Shared helpers for the GPU parity tests: move seeded inputs to the GPU,
run the HIP library through its binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

from oracle import muon_oracle as om

COEFFS = om.DEFAULT_COEFFS
LR = 0.02
BETA = 0.95
NS_TOL = 1e-2      # relative Frobenius error per matrix, Newton-Schulz outputs
MOM_TOL = 1e-6     # relative Frobenius error per matrix, fp32 momentum buffers


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_f(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    n = np.linalg.norm(y)
    d = np.linalg.norm(x - y)
    return d / n if n > 0 else d


def torch_mod():
    import torch
    return torch


def to_gpu(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_gpu(bits_u16):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def bf16_to_np(t):
    """bf16 torch tensor -> fp32 numpy (exact)."""
    torch = torch_mod()
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return om.bf16_to_f32(bits)


def empty_bf16(shape):
    torch = torch_mod()
    return torch.empty(shape, dtype=torch.bfloat16, device="cuda")


def gpu_step(mats, grads_key, steps, ns_steps=5, lr=LR, beta=BETA, coeffs=COEFFS, want_updates=True):
    """Run `steps` Muon steps on the GPU; mats is a list of dicts from
    workloads.make_matrix.  Returns (W list, buf list, last updates list)."""
    import optimizer_muon_step_amd as mu
    torch = torch_mod()
    W = [to_gpu(m["W"]) for m in mats]
    M = [to_gpu(m["buf"]) for m in mats]
    U = None
    for s in range(steps):
        G = [to_gpu(m[grads_key][s]) for m in mats]
        U = [empty_bf16(m["W"].shape) for m in mats] if want_updates else None
        mu.muon_step(W, G, M, lr, beta, ns_steps, coeffs, updates=U)
        del G
    torch.cuda.synchronize()
    return W, M, U


def oracle_steps(m, steps, ns_steps=5, lr=LR, beta=BETA, coeffs=COEFFS, grads_key="grads"):
    W, buf = m["W"], m["buf"]
    r = None
    for s in range(steps):
        r = om.muon_step_matrix(W, m[grads_key][s], buf, lr, beta, ns_steps, coeffs)
        W, buf = r["W"], r["buf"]
    return r


def check_matrix(tag, W_gpu, M_gpu, U_gpu, r_oracle, W_prev, ns_tol=NS_TOL):
    """Compare one matrix after a step: momentum, update and parameter delta."""
    w = W_gpu.cpu().numpy()
    m = M_gpu.cpu().numpy()
    e_mom = rel_f(m, r_oracle["buf"])
    e_upd = rel_f(bf16_to_np(U_gpu), r_oracle["O"]) if U_gpu is not None else 0.0
    e_dw = rel_f(w.astype(np.float64) - W_prev, r_oracle["W"].astype(np.float64) - W_prev)
    say(f"  {tag}: momentum relF {e_mom:.2e}  update relF {e_upd:.2e}  dW relF {e_dw:.2e}")
    assert e_mom <= MOM_TOL, f"{tag}: momentum relF {e_mom}"
    assert e_upd <= ns_tol, f"{tag}: update relF {e_upd}"
    assert e_dw <= ns_tol, f"{tag}: param delta relF {e_dw}"
    return e_mom, e_upd, e_dw
