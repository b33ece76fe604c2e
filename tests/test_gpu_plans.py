"""GPU checks of the plan cache and of the memory around caller buffers:
plans are keyed on shapes, so alternating pointer sets costs no new plan
and no synchronisation and still matches the oracle; and no kernel writes
outside the caller's matrices (sentinel-filled guard bands around every
array of edge shapes stay untouched)."""
import numpy as np
import pytest

from gpu_helpers import BETA, COEFFS, LR, bf16_to_np, check_matrix, oracle_steps, say, to_gpu, torch_mod
from optimizer_muon_step_amd import workloads as wl

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


def test_alternating_pointer_sets_match_oracle_without_replanning():
    """Two independent optimizer states on the same shapes (one GPT-2 block),
    stepped alternately for 10 calls: each call brings the other pointer set.
    After the first call the cache builds no plan and never synchronises; each
    state matches the oracle after its 5 steps."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    steps = 5
    A = [wl.make_matrix("c2", i, steps) for i in range(4)]
    B = [{"W": (m["W"] * np.float32(0.5)).astype(np.float32), "buf": m["buf"].copy(),
          "grads": list(reversed(m["grads"]))} for m in A]
    state = {}
    for tag, mats in (("A", A), ("B", B)):
        state[tag] = ([to_gpu(m["W"]) for m in mats], [to_gpu(m["buf"]) for m in mats])
    stats = []
    for call in range(2 * steps):
        tag, mats = (("A", A), ("B", B))[call % 2]
        W, M = state[tag]
        G = [to_gpu(m["grads"][call // 2]) for m in mats]
        mu.muon_step(W, G, M, LR, BETA, 5, COEFFS)
        torch.cuda.synchronize()
        stats.append(mu.muon_plan_stats())
    first, last = stats[0], stats[-1]
    say(f"  plan stats after call 1: {first}; after call 10: {last}")
    assert last["plan_builds"] == first["plan_builds"]
    assert last["device_syncs"] == first["device_syncs"]
    assert last["uploads"] == first["uploads"]
    assert last["pointer_patches"] == first["pointer_patches"] + 9  # every call switched sets
    for tag, mats in (("A", A), ("B", B)):
        W, M = state[tag]
        for i, m in enumerate(mats):
            r = oracle_steps(m, steps)
            w = W[i].cpu().numpy()
            check_matrix(f"set {tag} matrix {i}", W[i], M[i], None, r, m["W"].astype(np.float64))
            assert np.isfinite(w).all()


SENTINEL32 = np.uint32(0x7FBADBAD)  # a NaN no kernel produces
SENTINEL16 = np.uint16(0x7FBA)


def _guarded(torch, arr, margin, kind):
    """A caller array inside a larger buffer whose margins hold a sentinel.
    Returns (buffer, view) with the view carrying arr's values."""
    n = arr.size
    if kind == "f32":
        host = np.full(n + 2 * margin, SENTINEL32, np.uint32)
        host[margin:margin + n] = np.ascontiguousarray(arr, np.float32).reshape(-1).view(np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda()
        view = buf[margin:margin + n].view(torch.float32).view(arr.shape)
    else:
        host = np.full(n + 2 * margin, SENTINEL16, np.uint16)
        buf = torch.from_numpy(host.view(np.int16)).cuda()
        view = buf[margin:margin + n].view(torch.bfloat16).view(arr.shape)
    return buf, view


def _margins_intact(buf, margin, n, kind):
    host = buf.cpu().numpy()
    host = host.view(np.uint32) if kind == "f32" else host.view(np.uint16)
    s = SENTINEL32 if kind == "f32" else SENTINEL16
    return bool(np.all(host[:margin] == s) and np.all(host[margin + n:] == s))


# Edge shapes (large update tiles, medium Gram and poly tiles), and a
# mid-sized ragged set that takes the medium tiles for every kind.
GUARD_SETS = {
    "edge": [(50257, 768), (5, 4099), (257, 129), (129, 257), (1, 1), (300, 1)],
    "medium": [(768, 3072), (3072, 769), (257, 1000)],
}


@pytest.mark.parametrize("margin", [4096, 4097])
@pytest.mark.parametrize("shape_set", sorted(GUARD_SETS))
def test_guard_bands_around_edge_shapes(margin, shape_set):
    """Every W, G, momentum and update buffer sits between two
    sentinel-filled margins; after two steps the margins are untouched and the
    results match the oracle.  margin 4097 also makes every array start off
    16-byte alignment (scalar paths)."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(70 + margin)
    shapes = GUARD_SETS[shape_set]
    say(f"[guard bands] margin {margin} elements, shapes {shapes}")
    mats = []
    for s in shapes:
        g = [rng.standard_normal(s).astype(np.float32) for _ in range(2)]
        if s == (50257, 768):  # row-sparse like the embedding gradient
            for k in range(2):
                keep = np.zeros(s[0], bool)
                keep[rng.choice(s[0], 2000, replace=False)] = True
                g[k][~keep] = 0.0
                g[k] *= np.float32(1e-2)
        mats.append({"W": (rng.standard_normal(s) * 0.02).astype(np.float32), "buf": np.zeros(s, np.float32),
                     "grads": g})
    bufs = []
    W, M, U = [], [], []
    for m in mats:
        bw, w = _guarded(torch, m["W"], margin, "f32")
        bm, mm = _guarded(torch, m["buf"], margin, "f32")
        bu, u = _guarded(torch, np.zeros(m["W"].shape, np.float32), margin, "bf16")
        bufs += [(bw, m["W"].size, "f32"), (bm, m["W"].size, "f32"), (bu, m["W"].size, "bf16")]
        W.append(w)
        M.append(mm)
        U.append(u)
    for step in range(2):
        gb = []
        G = []
        for m in mats:
            b, g = _guarded(torch, m["grads"][step], margin, "f32")
            gb.append((b, m["W"].size, "f32"))
            G.append(g)
        mu.muon_step(W, G, M, LR, BETA, 5, COEFFS, updates=U)
        torch.cuda.synchronize()
        for b, n, kind in bufs + gb:
            assert _margins_intact(b, margin, n, kind), "a kernel wrote outside a caller array"
    for i, (s, m) in enumerate(zip(shapes, mats)):
        r = oracle_steps(m, 2)
        check_matrix(f"{s}", W[i], M[i], U[i], r, m["W"].astype(np.float64))
        assert bf16_to_np(U[i]).shape == s


def test_lanes_give_bit_identical_results():
    """The lanes only decide which stream a shape group's kernels run on:
    two steps on one GPT-2 block (three shape groups) with 1, 2 and 3 lanes
    give the same bits, and match the oracle."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    mats = [wl.make_matrix("c2", i, 2) for i in range(4)]
    outs = []
    try:
        for lanes in (1, 2, 3):
            mu.muon_set_lanes(lanes)
            W = [to_gpu(m["W"]) for m in mats]
            M = [to_gpu(m["buf"]) for m in mats]
            for step in range(2):
                mu.muon_step(W, [to_gpu(m["grads"][step]) for m in mats], M, LR, BETA, 5, COEFFS)
            torch.cuda.synchronize()
            outs.append((W, M))
    finally:
        mu.muon_set_lanes(1)
    for W, M in outs[1:]:
        for a, b in zip(W + M, outs[0][0] + outs[0][1]):
            assert torch.equal(a, b)
    for i, m in enumerate(mats):
        r = oracle_steps(m, 2)
        check_matrix(f"lanes matrix {i}", outs[2][0][i], outs[2][1][i], None, r, m["W"].astype(np.float64))
    with pytest.raises(mu.MuonError, match="EINVAL"):
        mu.muon_set_lanes(5)
