"""Graph capture: once a pointer set's plan is cached, a step only enqueues
kernel launches, so it can be captured into a HIP graph and replayed.  Each
replay must equal the eager step on copies of the same state, bit for bit,
with eager work and synchronisations between the replays."""
import numpy as np
import pytest

from gpu_helpers import COEFFS, say, to_gpu, torch_mod
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


# c1 runs the small tiles with poly and update in one launch, c2 the medium
# tiles with cut Gram tiles and their reduce pass.
@pytest.mark.parametrize("config,count", [("c1", 1), ("c2", 4)])
def test_captured_muon_step_replays_like_eager(config, count):
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    say(f"[graph] {config}")
    mats = [wl.make_matrix(config, i, 4) for i in range(count)]
    W = [to_gpu(m["W"]) for m in mats]
    M = [to_gpu(m["buf"]) for m in mats]
    G = [to_gpu(m["grads"][0]) for m in mats]
    We = [w.clone() for w in W]
    Me = [m.clone() for m in M]
    Ge = [g.clone() for g in G]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mu.muon_step(W, G, M, 0.02, 0.95, 5, COEFFS)  # builds and caches the plan for these pointers
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mu.muon_step(We, Ge, Me, 0.02, 0.95, 5, COEFFS)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mu.muon_step(W, G, M, 0.02, 0.95, 5, COEFFS)
    for rep in range(1, 4):
        # new gradients in place, eager work between replays
        for i, m in enumerate(mats):
            G[i].copy_(to_gpu(m["grads"][rep]))
            Ge[i].copy_(G[i])
        graph.replay()
        mu.muon_step(We, Ge, Me, 0.02, 0.95, 5, COEFFS)
        torch.cuda.synchronize()
        for a, b in zip(W + M, We + Me):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        say(f"  replay {rep}: bit-identical to eager")


def test_captured_adamw_step_replays_like_eager():
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(40)
    sizes = [768, 4099, 50257]
    P = [to_gpu(rng.standard_normal(n).astype(np.float32)) for n in sizes]
    G = [to_gpu(rng.standard_normal(n).astype(np.float32)) for n in sizes]
    U = [torch.zeros(n, device="cuda") for n in sizes]
    V = [torch.zeros(n, device="cuda") for n in sizes]
    Pe, Ge, Ue, Ve = ([t.clone() for t in L] for L in (P, G, U, V))
    wds = [0.0, 0.1, 0.1]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mu.muon_adamw_step(P, G, U, V, 1e-3, weight_decay=wds, step=1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mu.muon_adamw_step(Pe, Ge, Ue, Ve, 1e-3, weight_decay=wds, step=1)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mu.muon_adamw_step(P, G, U, V, 1e-3, weight_decay=wds, step=2)  # step is baked into the capture
    for rep in range(3):
        graph.replay()
        mu.muon_adamw_step(Pe, Ge, Ue, Ve, 1e-3, weight_decay=wds, step=2)
        torch.cuda.synchronize()
        for a, b in zip(P + U + V, Pe + Ue + Ve):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"


def test_capture_survives_other_calls_between_replays():
    """A captured step keeps its plan and workspace: between replays the
    program makes eager steps with other pointers on the same shapes, a
    larger call that grows the library's workspace, and enough other shape
    sets to evict every uncaptured plan.  Each replay still equals the eager
    step on copies of the same state, bit for bit."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    torch.cuda.synchronize()
    mu.muon_release()  # start from an empty cache, so that the larger call below grows the workspace
    mats = [wl.make_matrix("c2", i, 4) for i in range(4)]
    W = [to_gpu(m["W"]) for m in mats]
    M = [to_gpu(m["buf"]) for m in mats]
    G = [to_gpu(m["grads"][0]) for m in mats]
    We, Me, Ge = ([t.clone() for t in L] for L in (W, M, G))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mu.muon_step(W, G, M, 0.02, 0.95, 5, COEFFS)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mu.muon_step(We, Ge, Me, 0.02, 0.95, 5, COEFFS)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mu.muon_step(W, G, M, 0.02, 0.95, 5, COEFFS)
    rng = np.random.default_rng(41)
    before = mu.muon_plan_stats()
    for rep in range(1, 4):
        for i, m in enumerate(mats):
            G[i].copy_(to_gpu(m["grads"][rep]))
            Ge[i].copy_(G[i])
        # other work first: a larger call (rep 1: the workspace grows), then
        # nine small shape sets (evicting every plan no graph uses)
        if rep == 1:
            big = (2048, 6144)
            mu.muon_step([to_gpu(rng.standard_normal(big).astype(np.float32))],
                         [to_gpu(rng.standard_normal(big).astype(np.float32))],
                         [torch.zeros(big, device="cuda")], 0.02, 0.95, 5, COEFFS)
        for k in range(9):
            s = (40 + 8 * k + rep, 96)
            mu.muon_step([torch.zeros(s, device="cuda")], [torch.ones(s, device="cuda")],
                         [torch.zeros(s, device="cuda")], 0.02, 0.95, 5, COEFFS)
        graph.replay()
        mu.muon_step(We, Ge, Me, 0.02, 0.95, 5, COEFFS)
        torch.cuda.synchronize()
        for a, b in zip(W + M, We + Me):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        say(f"  replay {rep}: bit-identical to eager")
    after = mu.muon_plan_stats()
    say(f"  plan stats before the other calls: {before}; after: {after}")
    assert after["evictions"] > before["evictions"] and after["workspace_allocs"] > before["workspace_allocs"]


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_of_unseen_shapes_is_refused():
    """A capture must not allocate: a call whose plan does not exist yet fails
    with MUON_EINVAL and records nothing."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    s = (77, 333)
    W = torch.zeros(s, device="cuda")
    G = torch.ones(s, device="cuda")
    M = torch.zeros(s, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(mu.MuonError, match="EINVAL"):
        with torch.cuda.graph(graph):
            mu.muon_step([W], [G], [M], 0.02, 0.95, 5, COEFFS)
    torch.cuda.synchronize()
    mu.muon_step([W], [G], [M], 0.02, 0.95, 5, COEFFS)  # fine eagerly
    torch.cuda.synchronize()
    assert torch.isfinite(W).all() and W.abs().sum() > 0
