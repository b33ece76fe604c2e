"""GPU parity of the multi-tensor AdamW entry point against the CPU oracle.

Every operation is one fp32 rounding on both sides, in the same order, with
correctly rounded division and square root, so the bar is bit-exactness of
params, exp_avg and exp_avg_sq."""
import numpy as np
import pytest

from gpu_helpers import say, to_gpu, torch_mod
from oracle import adamw_oracle as ao
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


def _bits_equal(got, want, tag):
    got = np.ascontiguousarray(got, np.float32).view(np.uint32)
    want = np.ascontiguousarray(want, np.float32).view(np.uint32)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{tag}: {bad.size} of {got.size} differ, first at {bad[:5]}"


def _run_gpu(tensors, steps, lr, betas, eps, wds, first_step=1):
    """tensors: list of dicts p, g (list per step), u, v (numpy).  Returns
    the GPU p, u, v after `steps` calls."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    P = [to_gpu(t["p"]) for t in tensors]
    U = [to_gpu(t["u"]) for t in tensors]
    V = [to_gpu(t["v"]) for t in tensors]
    for s in range(steps):
        G = [to_gpu(t["g"][s]) for t in tensors]
        mu.muon_adamw_step(P, G, U, V, lr, betas, eps, wds, step=first_step + s)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in P], [x.cpu().numpy() for x in U], [x.cpu().numpy() for x in V]


def _run_oracle(tensors, steps, lr, betas, eps, wds, first_step=1):
    out = []
    for i, t in enumerate(tensors):
        p, u, v = t["p"], t["u"], t["v"]
        for s in range(steps):
            p, u, v = ao.adamw_step(p, t["g"][s], u, v, lr, betas[0], betas[1], eps, wds[i], first_step + s)
        out.append((p, u, v))
    return out


SIZES = [1, 3, 4, 5, 63, 4095, 4096, 4097, 12289, 100003, (7, 9), (33, 130)]


def _ragged(seed, steps, moments):
    rng = np.random.default_rng(seed)
    ts = []
    for sz in SIZES:
        shape = sz if isinstance(sz, tuple) else (sz,)
        t = {"p": rng.standard_normal(shape).astype(np.float32),
             "g": [(rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 1)).astype(np.float32)
                   for _ in range(steps)],
             "u": (rng.standard_normal(shape) * 1e-2 * moments).astype(np.float32),
             "v": (rng.random(shape) * 1e-3 * moments).astype(np.float32)}
        ts.append(t)
    return ts


@pytest.mark.parametrize("moments,first_step", [(0, 1), (1, 17)])
def test_adamw_ragged_sizes_bit_exact(moments, first_step):
    steps = 3
    ts = _ragged(30 + moments, steps, moments)
    wds = [0.0 if i % 3 else 0.1 for i in range(len(ts))]
    say(f"[adamw ragged] {len(ts)} tensors, {steps} steps from t={first_step}")
    got = _run_gpu(ts, steps, 1e-3, (0.9, 0.999), 1e-8, wds, first_step)
    want = _run_oracle(ts, steps, 1e-3, (0.9, 0.999), 1e-8, wds, first_step)
    for i, (w_p, w_u, w_v) in enumerate(want):
        _bits_equal(got[0][i], w_p, f"p[{i}]")
        _bits_equal(got[1][i], w_u, f"u[{i}]")
        _bits_equal(got[2][i], w_v, f"v[{i}]")


def test_adamw_unaligned_views_bit_exact():
    """Tensors that start one element into their storage take the
    element-by-element path."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(31)
    n = 10001
    host = {k: rng.standard_normal(n + 1).astype(np.float32) for k in ("p", "g", "u")}
    host["v"] = rng.random(n + 1).astype(np.float32) * np.float32(1e-3)
    dev = {k: to_gpu(v)[1:] for k, v in host.items()}
    assert dev["p"].data_ptr() % 16 != 0
    mu.muon_adamw_step([dev["p"]], [dev["g"]], [dev["u"]], [dev["v"]], 3e-4, (0.9, 0.95), 1e-6, 0.01, step=5)
    torch.cuda.synchronize()
    p, u, v = ao.adamw_step(host["p"][1:], host["g"][1:], host["u"][1:], host["v"][1:], 3e-4, 0.9, 0.95, 1e-6,
                            0.01, 5)
    _bits_equal(dev["p"].cpu().numpy(), p, "p")
    _bits_equal(dev["u"].cpu().numpy(), u, "u")
    _bits_equal(dev["v"].cpu().numpy(), v, "v")


@pytest.mark.parametrize("moments,step", [(False, 1), (True, 1000)])
def test_adamw_gpt2_set_bit_exact(moments, step):
    """The GPT-2-124M AdamW set (100 tensors, 39.5 M elements) in one call."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    specs = wl.adamw_specs_gpt2()
    say(f"[adamw gpt2] generating {len(specs)} tensors (moments={moments})")
    ts = [wl.make_adamw_tensor(i, s, step, moments) for i, s in enumerate(specs)]
    wds = [1e-2 if s.decayed else 0.0 for s in specs]
    P = [to_gpu(t["p"]) for t in ts]
    G = [to_gpu(t["g"]) for t in ts]
    U = [to_gpu(t["u"]) for t in ts]
    V = [to_gpu(t["v"]) for t in ts]
    mu.muon_adamw_step(P, G, U, V, 6e-4, (0.9, 0.999), 1e-8, wds, step=step)
    torch.cuda.synchronize()
    for i, t in enumerate(ts):
        p, u, v = ao.adamw_step(t["p"], t["g"], t["u"], t["v"], 6e-4, 0.9, 0.999, 1e-8, wds[i], step)
        _bits_equal(P[i].cpu().numpy(), p, f"{specs[i].name} p")
        _bits_equal(U[i].cpu().numpy(), u, f"{specs[i].name} u")
        _bits_equal(V[i].cpu().numpy(), v, f"{specs[i].name} v")


def test_adamw_special_values():
    """Zero, subnormal and overflowing gradients, and eps = 0 with a zero
    gradient (0/0): IEEE results on both sides, NaNs in the same places."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    g = np.array([0.0, 1e-42, -1e-40, 1e20, -3e25, 2.5, -0.0, 1e-3] * 9, np.float32)
    n = g.size
    rng = np.random.default_rng(32)
    p0 = rng.standard_normal(n).astype(np.float32)
    for eps in (1e-8, 0.0):
        z = np.zeros(n, np.float32)
        P, G, U, V = to_gpu(p0), to_gpu(g), to_gpu(z), to_gpu(z)
        mu.muon_adamw_step([P], [G], [U], [V], 1e-2, (0.9, 0.999), eps, 0.1, step=1)
        torch.cuda.synchronize()
        with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
            p, u, v = ao.adamw_step(p0, g, z, z, 1e-2, 0.9, 0.999, eps, 0.1, 1)
        for got, want, tag in ((P, p, "p"), (U, u, "u"), (V, v, "v")):
            got = got.cpu().numpy()
            assert np.array_equal(np.isnan(got), np.isnan(want)), tag
            ok = ~np.isnan(want)
            _bits_equal(got[ok], want[ok], f"{tag} eps={eps}")


def test_adamw_agrees_with_torch_adamw():
    """An independent implementation: torch.optim.AdamW in fp64 on the CPU,
    three steps; the fp32 GPU result agrees to fp32 rounding."""
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(33)
    shapes = [(3000,), (40, 70)]
    p0 = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [[rng.standard_normal(s).astype(np.float32) for s in shapes] for _ in range(3)]
    ref = [torch.tensor(p.astype(np.float64), requires_grad=True) for p in p0]
    opt = torch.optim.AdamW(ref, lr=1e-2, betas=(0.875, 0.9990234375), eps=2.0 ** -20, weight_decay=0.25)
    P = [to_gpu(p) for p in p0]
    U = [to_gpu(np.zeros(s, np.float32)) for s in shapes]
    V = [to_gpu(np.zeros(s, np.float32)) for s in shapes]
    for s in range(3):
        for r, g in zip(ref, grads[s]):
            r.grad = torch.tensor(g.astype(np.float64))
        opt.step()
        mu.muon_adamw_step(P, [to_gpu(g) for g in grads[s]], U, V, 1e-2, (0.875, 0.9990234375), 2.0 ** -20, 0.25,
                           step=s + 1)
    torch.cuda.synchronize()
    for r, p in zip(ref, P):
        want = r.detach().numpy()
        err = np.max(np.abs(p.cpu().numpy() - want) / (np.abs(want) + 1e-2))
        say(f"  vs torch AdamW: max rel err {err:.2e}")
        assert err < 1e-5


def test_adamw_empty_tensors_and_timing():
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(34)
    p0 = rng.standard_normal(5000).astype(np.float32)
    g = rng.standard_normal(5000).astype(np.float32)
    e = torch.empty(0, device="cuda")
    P, G = to_gpu(p0), to_gpu(g)
    U, V = torch.zeros(5000, device="cuda"), torch.zeros(5000, device="cuda")
    mu.muon_timing_enable(mu.KERNEL_ADAMW)
    mu.muon_adamw_step([e, P, e], [e, G, e], [e, U, e], [e, V, e], 1e-3, weight_decay=[0.5, 0.0, 0.5])
    ms, launches = mu.muon_timing_read()
    mu.muon_timing_enable(-1)
    assert launches == 1 and ms > 0
    p, _, _ = ao.adamw_step(p0, g, np.zeros(5000, np.float32), np.zeros(5000, np.float32), 1e-3)
    _bits_equal(P.cpu().numpy(), p, "p")


@pytest.mark.parametrize("shape,transpose", [((50257, 768), True), ((70, 130), True), ((1, 5), True),
                                             ((300, 7), False)])
def test_untie_copies_param_and_moments(shape, transpose):
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    rng = np.random.default_rng(shape[0] + shape[1])
    host = [rng.standard_normal(shape).astype(np.float32) for _ in range(3)]
    host[2] = np.abs(host[2])
    dev = [to_gpu(h) for h in host]
    say(f"[untie] {shape} transpose={transpose}")
    out = mu.muon_adamw_untie(*dev, transpose=transpose)
    torch.cuda.synchronize()
    want = ao.untie_state(*host, transpose)
    for o, w, tag in zip(out, want, ("param", "exp_avg", "exp_avg_sq")):
        assert tuple(o.shape) == w.shape
        _bits_equal(o.cpu().numpy(), w, tag)
    # the untied copy continues the shared trajectory (one AdamW step each)
    g = rng.standard_normal(shape).astype(np.float32)
    gd = to_gpu(g)
    gt = to_gpu(np.ascontiguousarray(g.T)) if transpose else to_gpu(g)
    mu.muon_adamw_step([dev[0]], [gd], [dev[1]], [dev[2]], 1e-3, step=50)
    mu.muon_adamw_step([out[0]], [gt], [out[1]], [out[2]], 1e-3, step=50)
    torch.cuda.synchronize()
    for a, b in zip(dev, out):
        b = b.t() if transpose else b
        assert torch.equal(a, b.contiguous())


def test_adamw_weight_decay_schedule_bit_exact():
    """lambda changing every step (a schedule), a tensor with a lambda of its
    own, tensors without decay, and a step where every lambda is zero."""
    rng = np.random.default_rng(35)
    sizes = [5000, 300, 4096, 777]
    schedule = [[0.1, 0.0, 0.1, 0.3], [0.05, 0.0, 0.05, 0.3], [0.2, 0.0, 0.2, 0.2], [0.0, 0.0, 0.0, 0.0],
                [0.1, 0.0, 0.1, 0.3]]
    ts = [{"p": rng.standard_normal(n).astype(np.float32),
           "g": [rng.standard_normal(n).astype(np.float32) for _ in schedule],
           "u": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)} for n in sizes]
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    P = [to_gpu(t["p"]) for t in ts]
    U = [to_gpu(t["u"]) for t in ts]
    V = [to_gpu(t["v"]) for t in ts]
    want = [(t["p"], t["u"], t["v"]) for t in ts]
    for s, wds in enumerate(schedule):
        mu.muon_adamw_step(P, [to_gpu(t["g"][s]) for t in ts], U, V, 1e-2, (0.9, 0.999), 1e-8, wds, step=s + 1)
        want = [ao.adamw_step(*want[i][:1], ts[i]["g"][s], *want[i][1:], 1e-2, 0.9, 0.999, 1e-8, wds[i], s + 1)
                for i in range(len(ts))]
    torch.cuda.synchronize()
    for i, (wp, wu, wv) in enumerate(want):
        _bits_equal(P[i].cpu().numpy(), wp, f"p[{i}]")
        _bits_equal(U[i].cpu().numpy(), wu, f"u[{i}]")
        _bits_equal(V[i].cpu().numpy(), wv, f"v[{i}]")
