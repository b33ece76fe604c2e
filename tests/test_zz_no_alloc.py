"""The allocation-free entry point (muon_step_noalloc) through the C ABI:
two calls in a row, the second on smaller matrices, each bit-identical to
muon_step on copies of the same inputs (same kernels, same storage points)
and within the parity bar of the oracle; a call larger than the static
scratch array is refused and changes nothing."""
import ctypes

import numpy as np
import pytest

from gpu_helpers import BETA, COEFFS, LR, NS_TOL, oracle_steps, rel_f, say, to_gpu, torch_mod
from optimizer_muon_step_amd import _lib
from optimizer_muon_step_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    yield
    torch.cuda.synchronize()


def _call(entry, W, G, M):
    torch = torch_mod()
    lib = _lib.load()
    shapes = _lib.shape_array([tuple(w.shape) for w in W])
    args = (_lib.ptr_array([w.data_ptr() for w in W]), _lib.ptr_array([g.data_ptr() for g in G]),
            _lib.ptr_array([m.data_ptr() for m in M]), shapes, len(W), LR, BETA, 5, _lib.float3(COEFFS),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return getattr(lib, entry)(*args)


def _inputs(shapes, seed):
    rng = np.random.default_rng(seed)
    mats = []
    for s in shapes:
        mats.append({"W": (rng.standard_normal(s) * 0.02).astype(np.float32), "buf": np.zeros(s, np.float32),
                     "grads": [(rng.standard_normal(s) * 1e-3).astype(np.float32)]})
    return mats


def test_noalloc_matches_muon_step_on_two_calls_in_a_row():
    torch = torch_mod()
    block = [(s.rows, s.cols) for s in wl.config_specs("c2")]  # one GPT-2-124M block
    small = [(256, 512), (300, 200), (5, 4099)]
    sets = [(block, _inputs(block, 80)), (small, _inputs(small, 81))]
    outs = []
    for shapes, mats in sets:
        ref = ([to_gpu(m["W"]) for m in mats], [to_gpu(m["grads"][0]) for m in mats], [to_gpu(m["buf"]) for m in mats])
        got = ([to_gpu(m["W"]) for m in mats], [to_gpu(m["grads"][0]) for m in mats], [to_gpu(m["buf"]) for m in mats])
        assert _call("muon_step", *ref) == 0, _lib.load().muon_last_error()
        assert _call("muon_step_noalloc", *got) == 0, _lib.load().muon_last_error()
        outs.append((shapes, mats, ref, got))
    torch.cuda.synchronize()  # both calls of the no-alloc entry were enqueued back to back
    for shapes, mats, ref, got in outs:
        for i, s in enumerate(shapes):
            assert torch.equal(got[0][i], ref[0][i]) and torch.equal(got[2][i], ref[2][i]), f"{s} differs"
            r = oracle_steps(mats[i], 1)
            e = rel_f(got[0][i].cpu().numpy().astype(np.float64) - mats[i]["W"], r["W"].astype(np.float64) - mats[i]["W"])
            say(f"  {s}: bit-identical to muon_step; dW relF vs oracle {e:.2e}")
            assert e <= NS_TOL


def test_noalloc_on_the_small_fused_path():
    """A call of small tiles with every m <= 256 (poly and update in one
    launch), after the medium-tile calls above: bit-identical to muon_step."""
    torch = torch_mod()
    shapes = [(256, 512), (100, 300)]
    mats = _inputs(shapes, 82)
    ref = ([to_gpu(m["W"]) for m in mats], [to_gpu(m["grads"][0]) for m in mats], [to_gpu(m["buf"]) for m in mats])
    got = ([to_gpu(m["W"]) for m in mats], [to_gpu(m["grads"][0]) for m in mats], [to_gpu(m["buf"]) for m in mats])
    assert _call("muon_step", *ref) == 0, _lib.load().muon_last_error()
    assert _call("muon_step_noalloc", *got) == 0, _lib.load().muon_last_error()
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        assert torch.equal(got[0][i], ref[0][i]) and torch.equal(got[2][i], ref[2][i]), f"{s} differs"


def test_noalloc_refuses_calls_beyond_the_scratch():
    torch = torch_mod()
    shapes = [(s.rows, s.cols) for s in wl.config_specs("c3")]  # 489 MiB of workspace
    W = [torch.zeros(s, device="cuda") for s in shapes]
    G = [torch.ones(s, device="cuda") for s in shapes]
    M = [torch.zeros(s, device="cuda") for s in shapes]
    rc = _call("muon_step_noalloc", W, G, M)
    msg = _lib.load().muon_last_error().decode()
    say(f"  rc {rc}: {msg}")
    assert rc == -2 and "static scratch" in msg
    torch.cuda.synchronize()
    assert all(float(w.abs().sum()) == 0.0 and float(m.abs().sum()) == 0.0 for w, m in zip(W, M))
