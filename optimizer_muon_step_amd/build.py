"""Build libmuon.so (the gfx950 HIP kernels and the C ABI) in place with
hipcc, and the plain C caller muon_c_example linked against it."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmuon.so")
C_EXAMPLE = os.path.join(HERE, "muon_c_example")
SOURCES = ["muon_api.hip", "muon_noalloc.hip", "plan_host.cpp", "kernels_tables.hip", "kernels_momentum.hip", "kernels_elementwise.hip",
           "kernels_ns.hip", "kernels_ns_gram.hip", "kernels_ns_fused.hip", "kernels_adamw.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # every fp32 multiply and add is rounded on its own (no fused multiply-add)
    "-ffp-contract=off",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source options on top of FLAGS.  The Gram kernel and the cast and apply
# passes are scheduled with LLVM's iterative register-pressure-minimising
# strategy: the same arithmetic in another instruction order (bit-identical
# results), and same-box timings per c3 Gram launch of 89.5 against 93.1 us;
# for the cast and apply passes it ties the default scheduler on c3 and c2
# and runs the apply over 192 GPT-2-XL-shaped matrices in 2358 against
# 2528 us.  The other kernels keep the default scheduler, which is faster for
# them (update 165 against 169 us, momentum 167 against 277 under that
# strategy).
_MINREG = ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]
# The AdamW pass takes the iterative ILP strategy: 188.1-188.3 against
# 190.8-190.9 us per launch on the GPT-2 AdamW set (same box), bit-identical.
SOURCE_FLAGS = {
    "kernels_ns_gram.hip": _MINREG,
    "kernels_elementwise.hip": _MINREG,
    "kernels_adamw.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}

# Sources of the update GEMM, whose hardware-counter profile is tied to them.
UPDATE_KERNEL_SOURCES = ["ns_gemm_tile.h", "kernels_ns.hip"]


def update_kernel_fingerprint() -> str:
    """sha256 over the update GEMM's sources and its per-source options."""
    h = hashlib.sha256()
    for name in UPDATE_KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    h.update(repr(FLAGS + SOURCE_FLAGS.get("kernels_ns.hip", [])).encode())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          source_flags: dict[str, list[str]] | None = None) -> str:
    """Compile every source for gfx950 (always recompiles, one object per
    source, in parallel) and link them into libmuon.so."""
    flags_of = SOURCE_FLAGS if source_flags is None else source_flags
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="muon_build_") as tmpdir:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc(), *FLAGS, *inc, *(extra or []), *flags_of.get(src, []), "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                     text=True)))
            objs.append(obj)
        failed = []
        for src, cmd, p in procs:
            log = p.communicate()[0]
            if p.returncode != 0:
                sys.stderr.write(log)
                failed.append(src)
            elif verbose and log.strip():
                sys.stderr.write(log)
        if failed:
            raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, out)
    if out == LIB:
        build_c_example(verbose)
    return out


def build_c_example(verbose: bool = False) -> str:
    """Compile csrc/c_example.c with the host C compiler against libmuon.so."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no host C compiler")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "c_example.c"), "-L", HERE, "-lmuon", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", C_EXAMPLE]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{cc} failed with exit code {res.returncode}")
    return C_EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
