"""Optimizer memory: the "new optimizer" thread (tweet 3/8) puts the new
optimizer at half of AdamW's optimizer memory.  The state each step carries
to the next is one fp32 momentum buffer per parameter for Muon (the
momentum[] argument of muon_step) against two fp32 moments for AdamW
(exp_avg[] and exp_avg_sq[] of muon_adamw_step).  Pinned by what the oracle
steps return and by the byte count on the GPT-2-124M hidden set.

That is the state, not the library's footprint: muon_step also keeps a
workspace across steps (bf16 iterates, A, B and norm partials), 513.1 MB on
that set, so its device memory beyond the parameters (339.7 + 513.1 MB) is
above AdamW's 679.5 MB of state.  The last test pins that figure."""
import numpy as np

from oracle import adamw_oracle as ao
from oracle import muon_oracle as om
from optimizer_muon_step_amd import _lib
from optimizer_muon_step_amd import workloads as wl


def _state_bytes_per_param():
    W = np.zeros((4, 6), np.float32)
    g = np.ones_like(W)
    r = om.muon_step_matrix(W, g, np.zeros_like(W), 0.02, 0.95, 1)
    muon_state = [r["buf"]]
    _, u, v = ao.adamw_step(W, g, np.zeros_like(W), np.zeros_like(W), 1e-3)
    adam_state = [u, v]
    return (sum(a.nbytes for a in muon_state) / W.size, sum(a.nbytes for a in adam_state) / W.size)


def test_muon_state_is_half_of_adamw():
    muon_bpp, adam_bpp = _state_bytes_per_param()
    assert (muon_bpp, adam_bpp) == (4.0, 8.0)
    n = sum(s.rows * s.cols for s in wl.config_specs("c3"))
    assert n == 84_934_656
    assert round(n * muon_bpp / 1e6, 1) == 339.7 and round(n * adam_bpp / 1e6, 1) == 679.5


def test_entry_points_take_that_state():
    # muon_step: params, grads, momentum (one state array); muon_adamw_step:
    # params, grads, exp_avg, exp_avg_sq (two state arrays)
    assert _lib.SIGNATURES["muon_step"][1][:3] == [_lib._PP] * 3
    assert _lib.SIGNATURES["muon_adamw_step"][1][:4] == [_lib._PP] * 4


def test_workspace_beside_the_state():
    """The workspace the step needs on the GPT-2-124M hidden set (host logic of
    the library, no GPU): 513.1 MB, so state plus workspace exceed AdamW's
    state there."""
    shapes = [(s.rows, s.cols) for s in wl.config_specs("c3")]
    import optimizer_muon_step_amd as mu
    ws = mu.muon_workspace_bytes(shapes)
    assert round(ws / 1e6, 1) == 513.1
    n = sum(r * c for r, c in shapes)
    assert n * 4 + ws > n * 8
