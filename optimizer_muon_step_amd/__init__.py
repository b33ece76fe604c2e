"""Muon optimizer step on MI355X: Python binding of libmuon.so.

Thin argument marshalling over the C ABI declared in include/muon.h; every
step of the computation runs in the library's HIP kernels.  Tensors are torch
tensors on the current HIP device: fp32 params/grads/momentum, bf16 for the
Newton-Schulz entry.  Calls enqueue on torch's current stream (or `stream`)
and return without synchronising.
"""
from __future__ import annotations

import ctypes

from . import _lib

__all__ = [
    "DEFAULT_COEFFS", "MuonError", "matrix_shape", "muon_step", "muon_step_noalloc", "muon_newton_schulz", "muon_adamw_step", "muon_adamw_untie",
    "muon_workspace_bytes",
    "muon_set_workspace", "muon_release", "muon_plan_stats", "muon_set_lanes", "muon_timing_enable", "muon_timing_read", "muon_last_error",
    "KERNEL_MOMENTUM", "KERNEL_CAST", "KERNEL_GRAM", "KERNEL_POLY", "KERNEL_UPDATE", "KERNEL_APPLY",
    "KERNEL_ADAMW",
]

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
KERNEL_MOMENTUM, KERNEL_CAST, KERNEL_GRAM, KERNEL_POLY, KERNEL_UPDATE, KERNEL_APPLY, KERNEL_ADAMW = range(7)
_CODES = {-1: "MUON_EINVAL", -2: "MUON_ENOMEM", -3: "MUON_EHIP"}


class MuonError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


def muon_last_error() -> str:
    return (_lib.load().muon_last_error() or b"").decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise MuonError(rc, muon_last_error())


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def matrix_shape(shape):
    """The matrix a parameter of rank >= 2 is orthogonalised as: its first
    dimension by the product of the others (for a convolution filter
    out x in x kh x kw, the out x (in kh kw) matrix of its im2col form).  A
    contiguous row-major tensor already is that matrix in memory."""
    shape = tuple(int(d) for d in shape)
    if len(shape) < 2:
        raise ValueError("rank >= 2 expected (1-D parameters belong to another optimizer)")
    cols = 1
    for d in shape[1:]:
        cols *= d
    return shape[0], cols


def _fp32_matrix(t, what):
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() < 2:
        raise ValueError(f"{what}: expected a tensor of rank >= 2 (1-D parameters belong to another optimizer)")
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous float32 tensor on the GPU")
    return t.data_ptr()


def _bf16_matrix(t, what):
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() < 2:
        raise ValueError(f"{what}: expected a tensor of rank >= 2")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous bfloat16 tensor on the GPU")
    return t.data_ptr()


def _coeff_arg(coeffs, ns_steps):
    """(is a schedule, ctypes float array): one (a, b, c) for every iteration,
    or ns_steps triples, triple k for iteration k."""
    rows = [list(c) if hasattr(c, "__len__") else None for c in coeffs]
    if all(r is None for r in rows):
        vals = [float(c) for c in coeffs]
        if len(vals) != 3:
            raise ValueError("coeffs: expected (a, b, c) or one (a, b, c) per iteration")
        return False, _lib.float3(vals)
    if any(r is None or len(r) != 3 for r in rows) or len(rows) != ns_steps:
        raise ValueError(f"coeffs schedule: expected {ns_steps} triples (a, b, c)")
    return True, _lib.float_array([float(v) for r in rows for v in r])


def muon_step(params, grads, momentum, lr=0.02, beta=0.95, ns_steps=5, coeffs=DEFAULT_COEFFS,
              updates=None, stream=None) -> None:
    """One Muon step over lists of fp32 tensors of rank >= 2 (params and
    momentum updated in place; rank > 2 is taken as the matrix_shape view).
    `coeffs` is one (a, b, c) or a schedule of ns_steps triples.  `updates`, if
    given, is a list of bf16 tensors (or None entries) of the params' shapes
    receiving the applied update."""
    n = len(params)
    if len(grads) != n or len(momentum) != n:
        raise ValueError("params, grads and momentum must have the same length")
    shapes = []
    for i, (p, g, m) in enumerate(zip(params, grads, momentum)):
        _fp32_matrix(p, f"params[{i}]"), _fp32_matrix(g, f"grads[{i}]"), _fp32_matrix(m, f"momentum[{i}]")
        if g.shape != p.shape or m.shape != p.shape:
            raise ValueError(f"matrix {i}: shapes differ")
        shapes.append(matrix_shape(p.shape))
    lib = _lib.load()
    P = _lib.ptr_array([p.data_ptr() for p in params])
    G = _lib.ptr_array([g.data_ptr() for g in grads])
    M = _lib.ptr_array([m.data_ptr() for m in momentum])
    S = _lib.shape_array(shapes)
    sched, C = _coeff_arg(coeffs, ns_steps)
    st = ctypes.c_void_p(_stream_handle(stream))
    if updates is None:
        if sched:
            rc = lib.muon_step_sched(P, G, M, S, n, float(lr), float(beta), int(ns_steps), C, None, st)
        else:
            rc = lib.muon_step(P, G, M, S, n, float(lr), float(beta), int(ns_steps), C, st)
    else:
        if len(updates) != n:
            raise ValueError("updates must have one entry per matrix")
        ptrs = []
        for i, u in enumerate(updates):
            if u is None:
                ptrs.append(None)
                continue
            _bf16_matrix(u, f"updates[{i}]")
            if u.shape != params[i].shape:
                raise ValueError(f"updates[{i}]: shape differs from params[{i}]")
            ptrs.append(u.data_ptr())
        U = _lib.ptr_array(ptrs)
        entry = lib.muon_step_sched if sched else lib.muon_step_ex
        rc = entry(P, G, M, S, n, float(lr), float(beta), int(ns_steps), C, U, st)
    _check(rc)


def muon_step_noalloc(params, grads, momentum, lr=0.02, beta=0.95, ns_steps=5, coeffs=DEFAULT_COEFFS,
                      stream=None) -> None:
    """muon_step for callers that cannot allocate device memory: workspace and
    tables in the library's static scratch array (MUON_NOALLOC_SCRATCH_BYTES
    per device); one fixed (a, b, c) triple."""
    n = len(params)
    if len(grads) != n or len(momentum) != n:
        raise ValueError("params, grads and momentum must have the same length")
    shapes = []
    for i, (p, g, m) in enumerate(zip(params, grads, momentum)):
        _fp32_matrix(p, f"params[{i}]"), _fp32_matrix(g, f"grads[{i}]"), _fp32_matrix(m, f"momentum[{i}]")
        if g.shape != p.shape or m.shape != p.shape:
            raise ValueError(f"matrix {i}: shapes differ")
        shapes.append(matrix_shape(p.shape))
    sched, C = _coeff_arg(coeffs, ns_steps)
    if sched:
        raise ValueError("muon_step_noalloc takes one (a, b, c) triple")
    rc = _lib.load().muon_step_noalloc(_lib.ptr_array([p.data_ptr() for p in params]),
                                       _lib.ptr_array([g.data_ptr() for g in grads]),
                                       _lib.ptr_array([m.data_ptr() for m in momentum]), _lib.shape_array(shapes), n,
                                       float(lr), float(beta), int(ns_steps), C,
                                       ctypes.c_void_p(_stream_handle(stream)))
    _check(rc)


def muon_newton_schulz(xs, outs, ns_steps=5, coeffs=DEFAULT_COEFFS, stream=None) -> None:
    """The Newton-Schulz core alone on bf16 matrices (no normalisation);
    `coeffs` is one (a, b, c) or a schedule of ns_steps triples."""
    n = len(xs)
    if len(outs) != n:
        raise ValueError("xs and outs must have the same length")
    shapes = []
    for i, (x, o) in enumerate(zip(xs, outs)):
        _bf16_matrix(x, f"xs[{i}]"), _bf16_matrix(o, f"outs[{i}]")
        if x.shape != o.shape:
            raise ValueError(f"matrix {i}: shapes differ")
        shapes.append(matrix_shape(x.shape))
    lib = _lib.load()
    sched, C = _coeff_arg(coeffs, ns_steps)
    entry = lib.muon_newton_schulz_sched if sched else lib.muon_newton_schulz
    rc = entry(_lib.ptr_array([x.data_ptr() for x in xs]), _lib.ptr_array([o.data_ptr() for o in outs]),
               _lib.shape_array(shapes), n, int(ns_steps), C, ctypes.c_void_p(_stream_handle(stream)))
    _check(rc)


def _fp32_flat(t, what):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a tensor")
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous float32 tensor on the GPU")
    return t.data_ptr()


def muon_adamw_step(params, grads, exp_avg, exp_avg_sq, lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                    step=1, stream=None) -> None:
    """One AdamW step over tensors of any shape (each contiguous fp32, taken
    flat); exp_avg and exp_avg_sq start at zero and `step` counts from 1.
    `weight_decay` is one value or one per tensor."""
    n = len(params)
    if not (len(grads) == len(exp_avg) == len(exp_avg_sq) == n):
        raise ValueError("params, grads, exp_avg and exp_avg_sq must have the same length")
    if hasattr(weight_decay, "__len__"):
        wds = [float(w) for w in weight_decay]
        if len(wds) != n:
            raise ValueError("weight_decay: expected one value or one per tensor")
    else:
        wds = [float(weight_decay)] * n
    ptrs = ([], [], [], [])
    numels = []
    for i in range(n):
        ts = (params[i], grads[i], exp_avg[i], exp_avg_sq[i])
        names = ("params", "grads", "exp_avg", "exp_avg_sq")
        for k, (t, name) in enumerate(zip(ts, names)):
            ptrs[k].append(_fp32_flat(t, f"{name}[{i}]"))
        if len({t.numel() for t in ts}) != 1:
            raise ValueError(f"tensor {i}: element counts differ")
        numels.append(params[i].numel())
    b1, b2 = betas
    rc = _lib.load().muon_adamw_step(*(_lib.ptr_array(p) for p in ptrs), _lib.int64_array(numels),
                                     _lib.float_array(wds), n, float(lr), float(b1), float(b2), float(eps),
                                     int(step), ctypes.c_void_p(_stream_handle(stream)))
    _check(rc)


def muon_adamw_untie(param, exp_avg, exp_avg_sq, transpose=False, stream=None):
    """Delayed untying: new (param, exp_avg, exp_avg_sq) tensors copied from
    a shared 2-D parameter and its AdamW moments, transposed if asked, so the
    untied parameter continues from the shared point.  Returns the three new
    tensors (allocated here, filled by the library on the stream)."""
    import torch
    for t, name in ((param, "param"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _fp32_flat(t, name)
        if t.dim() != 2 or t.shape != param.shape:
            raise ValueError(f"{name}: expected a 2-D tensor of the parameter's shape")
    rows, cols = param.shape
    shape = (cols, rows) if transpose else (rows, cols)
    out = [torch.empty(shape, dtype=torch.float32, device=param.device) for _ in range(3)]
    rc = _lib.load().muon_adamw_untie(param.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(),
                                      out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), rows, cols,
                                      1 if transpose else 0, ctypes.c_void_p(_stream_handle(stream)))
    _check(rc)
    return tuple(out)


def muon_workspace_bytes(shapes) -> int:
    lib = _lib.load()
    b = lib.muon_workspace_bytes(_lib.shape_array(shapes), len(shapes))
    if b == 0 and len(shapes) > 0:
        raise MuonError(-1, muon_last_error())
    return int(b)


def muon_set_workspace(ptr: int | None, nbytes: int = 0) -> None:
    _check(_lib.load().muon_set_workspace(ctypes.c_void_p(ptr or 0), int(nbytes)))


def muon_release() -> None:
    _lib.load().muon_release()


PLAN_STATS = ("plan_builds", "uploads", "pointer_patches", "device_syncs", "evictions", "workspace_allocs")


def muon_plan_stats() -> dict:
    """Counters of the current device's plan cache (diagnostics)."""
    arr = (ctypes.c_int64 * 6)()
    _check(_lib.load().muon_plan_stats(arr))
    return dict(zip(PLAN_STATS, (int(v) for v in arr)))


def muon_set_lanes(lanes: int) -> None:
    """Concurrency of a call: up to `lanes` shape groups run at once on the
    library's internal streams (1 = everything on the caller's stream)."""
    _check(_lib.load().muon_set_lanes(int(lanes)))


def muon_timing_enable(kernel: int) -> None:
    _check(_lib.load().muon_timing_enable(int(kernel)))


def muon_timing_read():
    """(total milliseconds, number of launches) of the timed kernel family since the last read."""
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    _check(_lib.load().muon_timing_read(ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value
