"""Pins for the AdamW oracle, each against something other than the oracle:
the values the pages print for their worked example, closed forms of the
bias correction and of the decoupled decay, invariances, and a brute-force
fp32 evaluation in exact rational arithmetic.  The mutation test at the end
plants plausible slips in copies of the oracle and checks a pin fails."""
import math
import os
from fractions import Fraction as F

import numpy as np
import pytest

from exact_fp import fp32 as fp32_exact, fp32_sqrt
from oracle import adamw_oracle as ao

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adam_worked_example.txt")
BOWL_A = np.array([1.0, 10.0])
BOWL_C = np.array([3.0, -1.0])


def _golden():
    rows = {"grad": {}, "theta": {}, "loss": {}, "decay": []}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        kind = line[0]
        if kind == "decay":
            rows["decay"].append((float(line[1]), line[2], int(line[3])))
        elif kind == "loss":
            rows["loss"][int(line[1])] = line[2]
        else:
            rows[kind][int(line[1])] = [float(x) for x in line[2:]]
    return rows


def _bowl_path(steps, adamw_step=None, **kw):
    step_fn = adamw_step or ao.adamw_step
    th = np.zeros(2)
    u = np.zeros(2)
    v = np.zeros(2)
    path, grads = [th], []
    for t in range(1, steps + 1):
        g = 2.0 * BOWL_A * (th - BOWL_C)
        grads.append(g)
        th, u, v = step_fn(th, g, u, v, 0.1, 0.9, 0.999, 1e-8, 0.0, t, mode="exact", **kw)
        path.append(th)
    return path, grads


def _loss(th):
    return float(np.sum(BOWL_A * (th - BOWL_C) ** 2))


def _sig_digits_match(x, printed):
    """x rounds to the printed significant digits."""
    digits = len(printed.lower().split("e")[0].replace("-", "").replace(".", "").lstrip("0"))
    return f"{x:.{digits - 1}e}" == f"{float(printed):.{digits - 1}e}"


def test_worked_example_matches_the_printed_values():
    gold = _golden()
    path, grads = _bowl_path(300)
    assert np.array_equal(grads[0], np.array(gold["grad"][1]))
    for t, want in gold["theta"].items():
        assert np.all(np.abs(path[t] - np.array(want)) < 5e-7), (t, path[t], want)
    for t, printed in gold["loss"].items():
        assert _sig_digits_match(_loss(path[t]), printed), (t, _loss(path[t]), printed)


def test_zero_gradient_decays_by_one_minus_lr_lambda():
    for lr, printed, halving in _golden()["decay"]:
        p = np.array([1.0, -3.0, 0.5])
        z = np.zeros(3)
        p1, u1, v1 = ao.adamw_step(p, z, z, z, lr, 0.9, 0.999, 1e-6, 1e-2, 1, mode="exact")
        f = p1[0]
        assert f"{f:.7f}" == printed
        assert np.allclose(p1, p * f, rtol=0, atol=1e-15)
        assert np.all(u1 == 0) and np.all(v1 == 0)
        assert round(math.log(2) / -math.log(f)) == halving
        # fp32: the factor is fp32(1 - fp32(lr * lambda)), applied once
        p32, _, _ = ao.adamw_step(p.astype(np.float32), z, z, z, lr, 0.9, 0.999, 1e-6, 1e-2, 1)
        want = np.float32(1) - np.float32(lr) * np.float32(1e-2)
        assert np.array_equal(p32, p.astype(np.float32) * want)


def test_first_step_moves_by_lr_g_over_abs_g_plus_eps():
    """t = 1: uhat = g and vhat = g^2, so the step is lr * g / (|g| + eps)."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal(64) * 10.0 ** rng.integers(-6, 4, 64)
    p = rng.standard_normal(64)
    z = np.zeros(64)
    for eps in (1e-8, 1e-3):
        p1, _, _ = ao.adamw_step(p, g, z, z, 0.05, 0.9, 0.999, eps, 0.0, 1, mode="exact")
        want = p - 0.05 * g / (np.abs(g) + eps)
        assert np.max(np.abs(p1 - want) / np.abs(p - want)) < 1e-13


def test_constant_gradient_is_exactly_bias_corrected():
    """The same g every step: uhat_t = g and vhat_t = g^2 for every t, so
    every step is the same (the derivation block's 'true weighted average')."""
    rng = np.random.default_rng(2)
    g = rng.standard_normal(32)
    p0 = rng.standard_normal(32)
    p, u, v = p0, np.zeros(32), np.zeros(32)
    for t in range(1, 41):
        p, u, v = ao.adamw_step(p, g, u, v, 0.01, 0.9, 0.999, 1e-8, 0.0, t, mode="exact")
        want = p0 - t * 0.01 * g / (np.abs(g) + 1e-8)
        assert np.max(np.abs(p - want)) < 1e-12 * t


def test_weight_decay_is_decoupled():
    """AdamW's step is the Adam step of the same gradients applied to the
    decayed parameters: theta_t = (1 - lr lambda) theta_{t-1} - Delta_t, with
    Delta_t the weight-decay-free step (which does not depend on theta)."""
    rng = np.random.default_rng(3)
    grads = [rng.standard_normal(16) for _ in range(12)]
    p0 = rng.standard_normal(16)
    lr, lam = 0.1, 0.3
    pa, ua, va = p0, np.zeros(16), np.zeros(16)
    pw, uw, vw = p0, np.zeros(16), np.zeros(16)
    for t, g in enumerate(grads, 1):
        pa_new, ua, va = ao.adamw_step(pa, g, ua, va, lr, 0.9, 0.999, 1e-8, 0.0, t, mode="exact")
        delta = pa - pa_new
        want = (1 - lr * lam) * pw - delta
        pw, uw, vw = ao.adamw_step(pw, g, uw, vw, lr, 0.9, 0.999, 1e-8, lam, t, mode="exact")
        assert np.max(np.abs(pw - want)) < 1e-14
        assert np.array_equal(uw, ua) and np.array_equal(vw, va)
        pa = pa_new


@pytest.mark.parametrize("mode", ["exact", "emul"])
def test_gradient_scale_invariance_bit_exact(mode):
    """Gradients times 2^k with eps = 0: uhat scales by 2^k and sqrt(vhat) by
    2^k exactly, so the path is bit-identical."""
    rng = np.random.default_rng(4)
    grads = [rng.standard_normal(40).astype(np.float32) for _ in range(6)]
    paths = []
    p0 = rng.standard_normal(40).astype(np.float32)
    for k in (0, 7, -9):
        p = p0
        u = np.zeros(40, np.float32)
        v = np.zeros(40, np.float32)
        path = []
        for t, g in enumerate(grads, 1):
            p, u, v = ao.adamw_step(p, g * np.float32(2.0 ** k), u, v, 1e-3, 0.9, 0.999, 0.0, 0.1, t, mode=mode)
            path.append(p)
        paths.append(path)
    for other in paths[1:]:
        for a, b in zip(paths[0], other):
            assert np.array_equal(a, b)


def _brute_force_fp32(p, g, u, v, lr, b1, b2, eps, lam, t):
    """Reading W3 evaluated element by element in exact rational arithmetic,
    rounding to fp32 after every operation."""
    r = fp32_exact
    lr, b1, b2, eps, lam = (float(np.float32(x)) for x in (lr, b1, b2, eps, lam))
    omb1, omb2 = r(1.0 - b1), r(1.0 - b2)
    bc1, bc2 = float(np.float32(1.0 - b1 ** t)), float(np.float32(1.0 - b2 ** t))
    decay = r(1 - F(r(F(lr) * F(lam))))
    out = []
    for pe, ge, ue, ve in zip(p, g, u, v):
        pe, ge, ue, ve = (F(float(x)) for x in (pe, ge, ue, ve))
        p1 = r(pe * F(decay))
        u1 = r(F(r(F(b1) * ue)) + F(r(F(omb1) * ge)))
        v1 = r(F(r(F(b2) * ve)) + F(r(F(r(F(omb2) * ge)) * ge)))
        uh = r(F(u1) / F(bc1))
        vh = r(F(v1) / F(bc2))
        den = r(F(fp32_sqrt(vh)) + F(eps))
        p2 = r(F(p1) - F(r(F(r(F(lr) * F(uh))) / F(den))))
        out.append((p2, u1, v1))
    return [np.array(c, np.float32) for c in zip(*out)]


def test_emul_equals_exact_rational_fp32_evaluation():
    rng = np.random.default_rng(6)
    n = 48
    p = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 3, n)).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.integers(-20, 10, n)).astype(np.float32)
    g[:3] = [0.0, 1e-40, -3e-42]  # zero and subnormal gradients
    u = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-4).astype(np.float32)
    for (lr, b1, b2, eps, lam, t) in [(1e-3, 0.9, 0.999, 1e-8, 0.1, 1), (6e-4, 0.9, 0.95, 1e-6, 0.0, 7),
                                      (0.3, 0.5, 0.7, 1e-3, 2.0, 123)]:
        got = ao.adamw_step(p, g, u, v, lr, b1, b2, eps, lam, t)
        want = _brute_force_fp32(p, g, u, v, lr, b1, b2, eps, lam, t)
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_emul_tracks_exact_within_fp32_error():
    """Same fp32-representable scalars on both sides: over 50 steps the fp32
    path stays within a small multiple of fp32 rounding of the fp64 one."""
    rng = np.random.default_rng(7)
    sc = [float(np.float32(x)) for x in (1e-2, 0.9, 0.999, 1e-8, 0.1)]
    p = rng.standard_normal(1000).astype(np.float32)
    pe, ue, ve = p.astype(np.float64), np.zeros(1000), np.zeros(1000)
    pf, uf, vf = p, np.zeros(1000, np.float32), np.zeros(1000, np.float32)
    for t in range(1, 51):
        g = rng.standard_normal(1000).astype(np.float32)
        pe, ue, ve = ao.adamw_step(pe, g, ue, ve, *sc, t, mode="exact")
        pf, uf, vf = ao.adamw_step(pf, g, uf, vf, *sc, t)
    ulp = 2.0 ** -23
    assert np.max(np.abs(pf - pe)) < 50 * ulp * np.max(np.abs(pe))
    assert np.max(np.abs(uf - ue)) < 50 * ulp * np.max(np.abs(ue))
    assert np.max(np.abs(vf - ve)) < 50 * ulp * np.max(np.abs(ve))


def test_step_must_count_from_one():
    z = np.zeros(2)
    with pytest.raises(ValueError):
        ao.adamw_step(z, z, z, z, 0.1, step=0)


def test_multi_tensor_is_per_tensor():
    rng = np.random.default_rng(8)
    shapes = [(3,), (4, 5), (7,)]
    ps = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    gs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    zs = [np.zeros(s, np.float32) for s in shapes]
    res = ao.adamw_multi(ps, gs, zs, zs, 1e-3, weight_decay=[0.1, 0.0, 0.5], step=2)
    for i, lam in enumerate([0.1, 0.0, 0.5]):
        want = ao.adamw_step(ps[i], gs[i], zs[i], zs[i], 1e-3, weight_decay=lam, step=2)
        for a, b in zip(res[i], want):
            assert np.array_equal(a, b)


def test_mutations_are_caught(monkeypatch):
    """Plausible slips planted in copies of the oracle each fail a pin."""
    real = ao.adamw_step

    def no_bias_correction(p, g, u, v, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                           mode="emul"):
        p, u, v = (np.asarray(x, np.float64) for x in (p, u, v))
        p = p * (1 - lr * weight_decay)
        u = beta1 * u + (1 - beta1) * g
        v = beta2 * v + (1 - beta2) * g * g
        return p - lr * u / (np.sqrt(v) + eps), u, v

    def coupled_l2(p, g, u, v, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1, mode="emul"):
        g = np.asarray(g, np.float64) + weight_decay * np.asarray(p, np.float64)
        return real(p, g, u, v, lr, beta1, beta2, eps, 0.0, step, mode="exact")

    def decay_after_step(p, g, u, v, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                         mode="emul"):
        p2, u2, v2 = real(p, g, u, v, lr, beta1, beta2, eps, 0.0, step, mode="exact")
        return p2 * (1 - lr * weight_decay), u2, v2

    def first_moment_squared(p, g, u, v, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                             mode="emul"):
        p, u, v = (np.asarray(x, np.float64) for x in (p, u, v))
        t = int(step)
        p = p * (1 - lr * weight_decay)
        u = beta1 * u + (1 - beta1) * g
        v = beta2 * v + (1 - beta2) * np.abs(g)
        return p - lr * (u / (1 - beta1 ** t)) / (np.sqrt(v / (1 - beta2 ** t)) + eps), u, v

    pins = [test_worked_example_matches_the_printed_values, test_first_step_moves_by_lr_g_over_abs_g_plus_eps,
            test_constant_gradient_is_exactly_bias_corrected, test_weight_decay_is_decoupled,
            test_zero_gradient_decays_by_one_minus_lr_lambda]
    for bad in (no_bias_correction, coupled_l2, decay_after_step, first_moment_squared):
        monkeypatch.setattr(ao, "adamw_step", bad)
        failed = 0
        for pin in pins:
            try:
                pin()
            except AssertionError:
                failed += 1
        assert failed >= 1, bad.__name__
    monkeypatch.undo()


@pytest.mark.parametrize("transpose", [False, True])
def test_untied_copy_continues_the_shared_trajectory(transpose):
    """The page's point: copying the weights and both moments lets the
    untied parameter continue exactly where the shared one was (its next
    step with the same gradient equals the shared tensor's next step, bit
    for bit, up to the layout), while restarting the moments from zero does
    not (the bias correction restarts and the momentum is lost)."""
    rng = np.random.default_rng(70)
    shape = (37, 11)
    p = rng.standard_normal(shape).astype(np.float32)
    u = (rng.standard_normal(shape) * 1e-2).astype(np.float32)
    v = (rng.random(shape) * 1e-3).astype(np.float32)
    g = rng.standard_normal(shape).astype(np.float32)
    t = 500
    shared = ao.adamw_step(p, g, u, v, 1e-3, 0.9, 0.999, 1e-8, 0.0, t)
    cp, cu, cv = ao.untie_state(p, u, v, transpose)
    assert cp.shape == (shape[::-1] if transpose else shape)
    gl = np.ascontiguousarray(g.T) if transpose else g
    untied = ao.adamw_step(cp, gl, cu, cv, 1e-3, 0.9, 0.999, 1e-8, 0.0, t)
    for a, b in zip(shared, untied):
        b = b.T if transpose else b
        assert np.array_equal(a.view(np.uint32), np.ascontiguousarray(b).view(np.uint32))
    z = np.zeros_like(cu)
    reset = ao.adamw_step(cp, gl, z, z, 1e-3, 0.9, 0.999, 1e-8, 0.0, t)
    assert not np.allclose(reset[0], untied[0], rtol=0, atol=1e-5)
    # the copies are independent buffers
    assert not any(np.shares_memory(a, b) for a, b in zip((cp, cu, cv), (p, u, v)))
