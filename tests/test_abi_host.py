"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/muon.h declares, and rejects invalid arguments
before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from optimizer_muon_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from optimizer_muon_step_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("muon_step", "muon_step_ex", "muon_newton_schulz", "muon_last_error", "muon_workspace_bytes",
                 "muon_set_workspace", "muon_release", "muon_timing_enable", "muon_timing_read"):
        assert want in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (muon_\w+)", out))
    assert set(declared_functions()) <= exported


def test_library_is_built_for_gfx950():
    out = subprocess.run(["/opt/rocm/bin/roc-obj-ls", _lib.LIB_PATH], capture_output=True, text=True)
    if out.returncode != 0:
        pytest.skip("roc-obj-ls unavailable")
    assert "gfx950" in out.stdout


def _step(lib, params, grads, moms, shapes, n, lr=0.02, beta=0.95, k=5, coeffs=(3.4445, -4.775, 2.0315)):
    return lib.muon_step(params, grads, moms, shapes, n, lr, beta, k, _lib.float3(coeffs) if coeffs else None, None)


def test_invalid_arguments_are_rejected_before_any_hip_call(lib):
    fake = _lib.ptr_array([0x10000])
    fake2 = _lib.ptr_array([0x20000])
    fake3 = _lib.ptr_array([0x30000])
    good = _lib.shape_array([(4, 4)])
    cases = [
        (dict(params=None, grads=fake2, moms=fake3, shapes=good, n=1), "NULL"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=None, n=1), "shapes"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=_lib.shape_array([(0, 4)]), n=1), ">= 1"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=_lib.shape_array([(1 << 16, 1 << 16)]), n=1), "2^31"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=-1), "outside"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, lr=float("inf")), "lr"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, beta=1.0), "beta"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, beta=-0.1), "beta"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, k=-1), "ns_steps"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, k=65), "ns_steps"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, coeffs=(1.0, float("nan"), 0.0)), "coeffs"),
        (dict(params=fake, grads=fake2, moms=fake3, shapes=good, n=1, coeffs=None), "coeffs"),
        (dict(params=fake, grads=fake2, moms=fake, shapes=good, n=1), "overlaps"),
        (dict(params=_lib.ptr_array([0x10002]), grads=fake2, moms=fake3, shapes=good, n=1), "aligned"),
        (dict(params=_lib.ptr_array([None]), grads=fake2, moms=fake3, shapes=good, n=1), "NULL"),
    ]
    for kw, msg in cases:
        rc = _step(lib, **kw)
        assert rc == -1, (kw, rc)
        assert msg in lib.muon_last_error().decode(), (msg, lib.muon_last_error())
    # overlapping ranges of different matrices
    two = _lib.shape_array([(4, 4), (4, 4)])
    rc = lib.muon_step(_lib.ptr_array([0x10000, 0x10020]), _lib.ptr_array([0x20000, 0x21000]),
                       _lib.ptr_array([0x30000, 0x31000]), two, 2, 0.02, 0.95, 5, _lib.float3((1, 0, 0)), None)
    assert rc == -1 and "overlaps" in lib.muon_last_error().decode()
    # n == 0 needs no device and succeeds
    assert _step(lib, None, None, None, None, 0) in (0, -1)
    assert lib.muon_step(fake, fake2, fake3, good, 0, 0.02, 0.95, 5, _lib.float3((1, 0, 0)), None) == 0


def test_newton_schulz_entry_validation(lib):
    x = _lib.ptr_array([0x10000])
    s = _lib.shape_array([(4, 4)])
    c = _lib.float3((3.4445, -4.775, 2.0315))
    assert lib.muon_newton_schulz(None, x, s, 1, 5, c, None) == -1
    assert lib.muon_newton_schulz(x, x, s, 1, -2, c, None) == -1
    assert lib.muon_newton_schulz(_lib.ptr_array([0x10001]), x, s, 1, 5, c, None) == -1
    assert "aligned" in lib.muon_last_error().decode()


def test_schedule_entries_validate_every_triple(lib):
    fake = _lib.ptr_array([0x10000])
    fake2 = _lib.ptr_array([0x20000])
    fake3 = _lib.ptr_array([0x30000])
    good = _lib.shape_array([(4, 4)])
    sched = [3.4445, -4.775, 2.0315] * 4
    bad = list(sched)
    bad[10] = float("inf")  # iteration 3's b
    rc = lib.muon_step_sched(fake, fake2, fake3, good, 1, 0.02, 0.95, 4, _lib.float_array(bad), None, None)
    assert rc == -1 and "coeffs[10]" in lib.muon_last_error().decode()
    rc = lib.muon_step_sched(fake, fake2, fake3, good, 1, 0.02, 0.95, 4, None, None, None)
    assert rc == -1 and "coeffs" in lib.muon_last_error().decode()
    rc = lib.muon_newton_schulz_sched(fake, fake, good, 1, 4, _lib.float_array(bad), None)
    assert rc == -1 and "coeffs[10]" in lib.muon_last_error().decode()
    # a schedule may be empty when there are no iterations; n = 0 needs no device
    assert lib.muon_step_sched(fake, fake2, fake3, good, 0, 0.02, 0.95, 0, None, None, None) == 0
    assert lib.muon_step_sched(fake, fake2, fake3, good, 0, 0.02, 0.95, 4, _lib.float_array(sched), None,
                               None) == 0
    # the fixed-triple entries still require their triple
    rc = lib.muon_step(fake, fake2, fake3, good, 1, 0.02, 0.95, 0, None, None)
    assert rc == -1 and "coeffs" in lib.muon_last_error().decode()


def test_adamw_validation_before_any_hip_call(lib):
    P = [_lib.ptr_array([0x10000 * (k + 1)]) for k in range(4)]
    n1 = _lib.int64_array([64])

    def call(ptrs=P, numels=n1, wd=None, n=1, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, step=1):
        return lib.muon_adamw_step(*ptrs, numels, wd, n, lr, b1, b2, eps, step, None)

    cases = [
        (dict(step=0), "step"),
        (dict(b1=1.0), "beta1"),
        (dict(b2=-0.1), "beta2"),
        (dict(eps=-1e-8), "eps"),
        (dict(eps=float("nan")), "eps"),
        (dict(lr=float("inf")), "lr"),
        (dict(wd=_lib.float_array([-0.1])), "weight_decay[0]"),
        (dict(numels=_lib.int64_array([-1])), "numels[0]"),
        (dict(n=-1), "n = -1"),
        (dict(ptrs=[P[0], P[1], P[2], _lib.ptr_array([0])]), "exp_avg_sq[0] is NULL"),
        (dict(ptrs=[P[0], P[1], P[2], _lib.ptr_array([0x10002])]), "4-byte aligned"),
        (dict(ptrs=[P[0], P[1], P[2], _lib.ptr_array([0x10000 + 128])]), "overlaps"),
    ]
    for kw, msg in cases:
        assert call(**kw) == -1, kw
        assert msg in lib.muon_last_error().decode(), (kw, lib.muon_last_error())
    # no tensors, or only empty ones (whose pointers may be NULL): nothing to do, no device needed
    assert call(n=0) == 0
    nul = _lib.ptr_array([0])
    assert call(ptrs=[nul] * 4, numels=_lib.int64_array([0])) == 0


def test_untie_validation_before_any_hip_call(lib):
    src = [0x100000, 0x200000, 0x300000]
    dst = [0x400000, 0x500000, 0x600000]

    def call(s=src, d=dst, rows=64, cols=32, tr=1):
        return lib.muon_adamw_untie(*s, *d, rows, cols, tr, None)

    cases = [
        (dict(rows=0), "rows = 0"),
        (dict(cols=-3), "cols = -3"),
        (dict(rows=1 << 30, cols=1 << 20), "2^40"),
        (dict(tr=2), "transpose = 2"),
        (dict(s=[0, src[1], src[2]]), "NULL"),
        (dict(d=[dst[0], dst[1] + 2, dst[2]]), "4-byte aligned"),
        (dict(d=[dst[0], dst[0] + 1024, dst[2]]), "overlaps"),
        (dict(s=[src[0], dst[2] - 512, src[2]]), "exp_avg overlaps new_exp_avg_sq"),
    ]
    for kw, msg in cases:
        assert call(**kw) == -1, kw
        assert msg in lib.muon_last_error().decode(), (kw, lib.muon_last_error())


def test_matrix_shape_of_higher_rank():
    import optimizer_muon_step_amd as mu
    assert mu.matrix_shape((64, 32, 3, 3)) == (64, 288)
    assert mu.matrix_shape((5, 7)) == (5, 7)
    with pytest.raises(ValueError):
        mu.matrix_shape((9,))


def test_binding_coefficient_forms():
    import optimizer_muon_step_amd as mu
    sched, arr = mu._coeff_arg([(1, 2, 3), (4, 5, 6)], 2)
    assert sched and list(arr) == [1, 2, 3, 4, 5, 6]
    sched, arr = mu._coeff_arg((1, 2, 3), 7)
    assert not sched and list(arr) == [1, 2, 3]
    with pytest.raises(ValueError):
        mu._coeff_arg([(1, 2, 3)], 2)
    with pytest.raises(ValueError):
        mu._coeff_arg([(1, 2)], 1)


def test_workspace_bytes_host_logic(lib):
    def ws(shapes):
        return lib.muon_workspace_bytes(_lib.shape_array(shapes), len(shapes))
    assert ws([]) > 0  # control block only
    base = ws([])
    # bf16 ping-pong iterate + Gram + polynomial matrices, canonical and padded to 128
    one = ws([(768, 2304)]) - base
    assert one >= 2 * 768 * 2304 * 2 + 2 * 768 * 768 * 2
    assert ws([(2304, 768)]) - base == one  # orientation does not matter
    assert ws([(100, 200)]) - base >= 2 * 128 * 256 * 2 + 2 * 128 * 128 * 2
    # two small calls stay small together (16 update tiles): no Gram tile is cut
    assert ws([(768, 768), (256, 512)]) == ws([(768, 768)]) + ws([(256, 512)]) - base
    assert lib.muon_workspace_bytes(_lib.shape_array([(0, 3)]), 1) == 0
    assert "shape" in lib.muon_last_error().decode()


def test_workspace_bytes_long_k_gram_split(lib):
    """In a call of more than 40 update tiles (192 x 256) whose longest Gram
    tile K is more than twice the call's per-CU share (total tile K slices /
    256 CUs, at least 8), every Gram tile longer than the share is cut into K
    chunks of about the share, one fp32 partial tile each: the only workspace term that depends on the other
    matrices of the call.  The Gram tiles are 256 x 256 in calls of at least
    256 such tiles, else 128 x 128 (their partial tiles too).  Calls of at
    most 40 update tiles and no Gram K over 32 slices run the small-tile
    kernels and cut nothing."""
    def ws(shapes):
        return lib.muon_workspace_bytes(_lib.shape_array(shapes), len(shapes))
    base = ws([])
    part, part_med = 256 * 256 * 4, 128 * 128 * 4
    a = (256, 65536)   # one Gram tile of 1024 K slices (three of 128); 512 update tiles
    b = (2048, 2048)   # 36 Gram tiles of 32 slices (136 of 128); 88 update tiles
    d = (64, 4100)     # one Gram tile of 65 slices; 34 update tiles, but K over 32 slices: not small
    e = (64, 2048)     # one Gram tile of 32 slices; 16 update tiles: a small call alone
    # a or d with eight b: 289 Gram tiles of 256, share ceil((1024 + 8 *
    # 1152) / 256) = 40 (a cut into ceil(1024 / 40) = 26 chunks, b's tiles of
    # 32 <= 80 not cut) and ceil((65 + 9216) / 256) = 37 (d's 65 <= 74 not
    # cut); eight b alone: 288 tiles of 256, share 36, nothing cut
    core_a = ws([a] + [b] * 8) - ws([b] * 8) - 26 * part
    core_d = ws([d] + [b] * 8) - ws([b] * 8)
    core_e = ws([e] + [b] * 8) - ws([b] * 8)  # share 37: e's 32 slices not cut
    core_b = (ws([b] * 8) - base) // 8
    assert core_a > 2 * 256 * 65536 * 2 and core_b > 2 * 2048 * 2048 * 2
    # a alone: three Gram tiles of 128, share max(8, 3072 / 256) = 12, each
    # tile in ceil(1024 / 12) = 86 chunks
    assert ws([a]) - base == core_a + 3 * 86 * part_med
    # b alone: 136 tiles of 128, share ceil(4352 / 256) = 17; 32 <= 34, nothing cut
    assert ws([b]) - base == core_b
    # d alone: three Gram tiles of 128, share 8, each in ceil(65 / 8) = 9 chunks
    assert ws([d]) - base == core_d + 3 * 9 * part_med
    # e alone is small: nothing cut
    assert ws([e]) - base == core_e
    # a with one b: tiles of 128, share ceil((3072 + 4352) / 256) = 29, and
    # a's 1024 > 58, so every tile longer than 29 is cut: each of a's in
    # ceil(1024 / 29) = 36 chunks, each of b's 136 in ceil(32 / 29) = 2
    assert ws([a, b]) - base == core_a + core_b + (3 * 36 + 136 * 2) * part_med


def test_timing_enable_validation(lib):
    assert lib.muon_timing_enable(99) == -1
    assert lib.muon_timing_enable(-1) == 0
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    assert lib.muon_timing_read(ctypes.byref(ms), ctypes.byref(cnt)) == 0 and cnt.value == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()
