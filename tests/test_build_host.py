"""Build configuration (CPU only): every per-source option names a compiled
source, the update kernel's fingerprint covers its sources and options, and
the built library carries a code object for gfx950."""
import os

import pytest

from optimizer_muon_step_amd import build as b


def test_source_flags_name_compiled_sources():
    for src in b.SOURCE_FLAGS:
        assert src in b.SOURCES, src
    for src in b.SOURCES + b.UPDATE_KERNEL_SOURCES:
        assert os.path.exists(os.path.join(b.CSRC, src)), src


def test_update_fingerprint_tracks_options(monkeypatch):
    f0 = b.update_kernel_fingerprint()
    assert f0 == b.update_kernel_fingerprint()
    monkeypatch.setitem(b.SOURCE_FLAGS, "kernels_ns.hip", ["-mllvm", "-some-option"])
    assert b.update_kernel_fingerprint() != f0
    monkeypatch.delitem(b.SOURCE_FLAGS, "kernels_ns.hip")
    assert b.update_kernel_fingerprint() == f0
    # options of other sources do not touch the update kernel
    monkeypatch.setitem(b.SOURCE_FLAGS, "kernels_momentum.hip", ["-mllvm", "-some-option"])
    assert b.update_kernel_fingerprint() == f0


def test_library_holds_gfx950_code():
    if not os.path.exists(b.LIB):
        pytest.skip("libmuon.so not built")
    with open(b.LIB, "rb") as f:
        data = f.read()
    assert b".hip_fatbin" in data                   # the device-code section
    assert b"amdgcn-amd-amdhsa--gfx950" in data     # a code object for gfx950
