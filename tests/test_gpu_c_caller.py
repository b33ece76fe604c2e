"""The C ABI without Python: the plain C program built with the library
(optimizer_muon_step_amd/csrc/c_example.c) runs one Muon step on matrices
read from a file, with its own device allocations and stream.  Its new
parameters, momentum and bf16 updates must equal, bit for bit, the same step
taken through the Python binding."""
import os
import struct
import subprocess

import numpy as np
import pytest

from gpu_helpers import BETA, COEFFS, LR, say, to_gpu, torch_mod

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "optimizer_muon_step_amd", "muon_c_example")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import optimizer_muon_step_amd as mu
    mu._lib.load()
    yield
    torch.cuda.synchronize()


def test_c_caller_matches_python_binding(tmp_path):
    torch = torch_mod()
    import optimizer_muon_step_amd as mu
    assert os.path.exists(EXE), "muon_c_example is built with the library (__graft_entry__.build())"
    shapes = [(256, 512), (700, 300), (33, 1000), (1, 1)]
    rng = np.random.default_rng(5)
    mats = [(rng.standard_normal(s).astype(np.float32) * np.float32(0.02), rng.standard_normal(s).astype(np.float32),
             rng.standard_normal(s).astype(np.float32) * np.float32(0.1)) for s in shapes]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("=iffi3f", len(shapes), LR, BETA, 5, *COEFFS))
        for r, c in shapes:
            f.write(struct.pack("=qq", r, c))
        for W, G, M in mats:
            f.write(W.tobytes() + G.tobytes() + M.tobytes())
    say(f"[c caller] {shapes}")
    subprocess.run([EXE, str(src), str(dst)], check=True, timeout=120)
    out = np.fromfile(dst, dtype=np.uint8)

    W = [to_gpu(w) for w, _, _ in mats]
    G = [to_gpu(g) for _, g, _ in mats]
    M = [to_gpu(m) for _, _, m in mats]
    U = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    mu.muon_step(W, G, M, LR, BETA, 5, COEFFS, updates=U)
    torch.cuda.synchronize()

    pos = 0
    for i, (r, c) in enumerate(shapes):
        e = r * c
        w_c = out[pos:pos + 4 * e].view(np.float32).reshape(r, c)
        m_c = out[pos + 4 * e:pos + 8 * e].view(np.float32).reshape(r, c)
        u_c = out[pos + 8 * e:pos + 10 * e].view(np.uint16).reshape(r, c)
        pos += 10 * e
        assert np.array_equal(w_c, W[i].cpu().numpy()), f"matrix {i}: params differ"
        assert np.array_equal(m_c, M[i].cpu().numpy()), f"matrix {i}: momentum differs"
        assert np.array_equal(u_c, U[i].view(torch.int16).cpu().numpy().view(np.uint16)), f"matrix {i}: update differs"
    assert pos == out.size
