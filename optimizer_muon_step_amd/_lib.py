"""ctypes loader for libmuon.so (argument types only; no computation here)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

# Entry points declared in include/muon.h, with their ctypes signatures.
_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


class MuonShape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_SHAPES = ctypes.POINTER(MuonShape)
_FLOAT3 = ctypes.POINTER(ctypes.c_float)

SIGNATURES = {
    "muon_step": (ctypes.c_int, [_PP, _PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_int, _FLOAT3, _P]),
    "muon_step_ex": (ctypes.c_int, [_PP, _PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_int, _FLOAT3, _PP, _P]),
    "muon_step_noalloc": (ctypes.c_int, [_PP, _PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_int, _FLOAT3, _P]),
    "muon_step_sched": (ctypes.c_int, [_PP, _PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int, _FLOAT3, _PP, _P]),
    "muon_newton_schulz": (ctypes.c_int, [_PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_int, _FLOAT3, _P]),
    "muon_newton_schulz_sched": (ctypes.c_int, [_PP, _PP, _SHAPES, ctypes.c_int, ctypes.c_int, _FLOAT3, _P]),
    "muon_adamw_step": (ctypes.c_int, [_PP, _PP, _PP, _PP, ctypes.POINTER(ctypes.c_int64), _FLOAT3, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int64, _P]),
    "muon_adamw_untie": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _P]),
    "muon_last_error": (ctypes.c_char_p, []),
    "muon_workspace_bytes": (ctypes.c_size_t, [_SHAPES, ctypes.c_int]),
    "muon_set_workspace": (ctypes.c_int, [_P, ctypes.c_size_t]),
    "muon_release": (None, []),
    "muon_plan_stats": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int64)]),
    "muon_set_lanes": (ctypes.c_int, [ctypes.c_int]),
    "muon_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "muon_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m optimizer_muon_step_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def shape_array(shapes):
    arr = (MuonShape * max(1, len(shapes)))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows = int(r)
        arr[i].cols = int(c)
    return arr


def float3(vals):
    arr = (ctypes.c_float * 3)()
    for i, v in enumerate(vals):
        arr[i] = float(v)
    return arr


def float_array(vals):
    arr = (ctypes.c_float * max(1, len(vals)))()
    for i, v in enumerate(vals):
        arr[i] = float(v)
    return arr


def int64_array(vals):
    arr = (ctypes.c_int64 * max(1, len(vals)))()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr
