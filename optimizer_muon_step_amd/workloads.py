"""Seeded synthetic inputs for the Muon step: GPT-2-shaped parameter,
gradient and momentum matrices.

This module only draws random numbers; it holds none of the optimizer's
arithmetic.  Both the HIP path and the CPU oracle are fed from it, so the two
sides always see the same fp32 bytes.

Every matrix has its own seed (config seed, matrix index, role), so any single
matrix of a large configuration can be regenerated alone, e.g. to check a
sample of a 1.47 B-parameter set on the CPU.

Workloads (shapes are listed rows x cols, in the in x out orientation GPT-2's
Conv1D weights use; the GPT-2 width 768 / 12 layers / 12 heads and the 1024
context come from the GPT-2 reproduction pages, the matrix factors 3x and 4x
and the XL width 1600 / 48 layers are the standard GPT-2 family shapes):

  c1  one 256 x 512 gradient, N(0, 1)
  c2  one GPT-2-124M block: 768x2304, 768x768, 768x3072, 3072x768;
      N(0, 1e-3^2) noise plus a rank-4 spike whose Frobenius norm is 10x the
      noise's
  c3  the full GPT-2-124M hidden set: 12 layers x the four c2 shapes,
      N(0, 1e-3^2) times a per-layer factor 10^U, U ~ U(-1, 1)
  c4  a GPT-2-XL-shaped hidden set: 48 layers x 1600x4800, 1600x1600,
      1600x6400, 6400x1600, same distribution as c3
  c5  stress: 50257x768 with only 2000 random rows non-zero (N(0, 1e-2^2)),
      the embedding-gradient sparsity the delayed-untying article describes;
      plus a 768x768 matrix with singular values log-spaced from 1e-6 to 1

Initial parameters are N(0, 0.02^2) (GPT-2's init std); momentum starts at 0.

AdamW workload (the GPT-2-124M parameters outside the hidden set, which the
thread's replies route to AdamW): the token embedding 50257x768 (tied with
the output layer) and the position embedding 1024x768, weight-decayed; per
layer the two LayerNorm gains and biases (768 each) and the four linear
biases (2304, 768, 3072, 768), and the final LayerNorm's gain and bias, all
1-D and not decayed (the GPT-2 lecture pages decay matrices, not 1-D
parameters).  100 tensors, 39,505,152 elements.  Parameters N(0, 0.02^2),
gradients N(0, 1e-3^2) per tensor scaled by 10^U, U ~ U(-1, 1); for a
mid-training step the moments are drawn too (exp_avg N(0, 1e-3^2), exp_avg_sq
the square of another such draw).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GPT2_WIDTH = 768
GPT2_LAYERS = 12
GPT2XL_WIDTH = 1600
GPT2XL_LAYERS = 48
VOCAB = 50257


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    layer: int
    kind: str  # "gauss", "spike", "layer_scaled", "row_sparse", "ill_cond"


def _block_shapes(width):
    return [(width, 3 * width), (width, width), (width, 4 * width), (4 * width, width)]


CONFIG_INDEX = {"c1": 0, "c2": 1, "c3": 2, "c4": 3, "c5": 4}


def config_specs(name: str) -> list[MatrixSpec]:
    if name == "c1":
        return [MatrixSpec(256, 512, 0, "gauss")]
    if name == "c2":
        return [MatrixSpec(r, c, 0, "spike") for r, c in _block_shapes(GPT2_WIDTH)]
    if name == "c3":
        return [MatrixSpec(r, c, layer, "layer_scaled")
                for layer in range(GPT2_LAYERS) for r, c in _block_shapes(GPT2_WIDTH)]
    if name == "c4":
        return [MatrixSpec(r, c, layer, "layer_scaled")
                for layer in range(GPT2XL_LAYERS) for r, c in _block_shapes(GPT2XL_WIDTH)]
    if name == "c5":
        return [MatrixSpec(VOCAB, GPT2_WIDTH, 0, "row_sparse"),
                MatrixSpec(GPT2_WIDTH, GPT2_WIDTH, 0, "ill_cond")]
    raise ValueError(f"unknown workload {name!r}")


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _seed(name: str) -> int:
    return 1000 + CONFIG_INDEX[name]


def _orthonormal(rng, n, k):
    """n x k with orthonormal columns (QR of a Gaussian, signs fixed so the
    distribution is Haar)."""
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def layer_factor(name: str, layer: int) -> float:
    u = _rng(_seed(name), 1 << 20, layer).uniform(-1.0, 1.0)
    return float(10.0 ** u)


def make_params(name: str, idx: int, spec: MatrixSpec) -> np.ndarray:
    rng = _rng(_seed(name), idx, 0)
    w = rng.standard_normal((spec.rows, spec.cols), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def make_grad(name: str, idx: int, spec: MatrixSpec, step: int = 1) -> np.ndarray:
    """Gradient of matrix `idx` for optimizer step `step` (1-based)."""
    rng = _rng(_seed(name), idx, step)
    r, c = spec.rows, spec.cols
    if spec.kind == "gauss":
        return rng.standard_normal((r, c), dtype=np.float32)
    if spec.kind == "layer_scaled":
        g = rng.standard_normal((r, c), dtype=np.float32)
        g *= np.float32(1e-3 * layer_factor(name, spec.layer))
        return g
    if spec.kind == "spike":
        noise = rng.standard_normal((r, c)) * 1e-3
        u = _orthonormal(rng, r, 4)
        v = _orthonormal(rng, c, 4)
        # ||U V^T||_F = 2 for orthonormal U, V with 4 columns
        amp = 10.0 * np.linalg.norm(noise) / 2.0
        return (noise + amp * (u @ v.T)).astype(np.float32)
    if spec.kind == "row_sparse":
        g = np.zeros((r, c), np.float32)
        rows = rng.choice(r, size=2000, replace=False)
        g[rows] = rng.standard_normal((2000, c), dtype=np.float32) * np.float32(1e-2)
        return g
    if spec.kind == "ill_cond":
        n = r
        u = _orthonormal(rng, n, n)
        v = _orthonormal(rng, n, n)
        sig = 10.0 ** (-6.0 + 6.0 * np.arange(n) / (n - 1))
        return ((u * sig) @ v.T).astype(np.float32)
    raise ValueError(spec.kind)


def make_matrix(name: str, idx: int, steps: int = 1) -> dict:
    """Inputs for one matrix: params W0, zero momentum, and `steps` gradients."""
    spec = config_specs(name)[idx]
    return {
        "spec": spec,
        "W": make_params(name, idx, spec),
        "buf": np.zeros((spec.rows, spec.cols), np.float32),
        "grads": [make_grad(name, idx, spec, s + 1) for s in range(steps)],
    }


def n_params(name: str) -> int:
    return sum(s.rows * s.cols for s in config_specs(name))


# ------------------------------------------------------------------ AdamW --

ADAMW_SEED = 2000


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    decayed: bool

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n


def adamw_specs_gpt2() -> list[TensorSpec]:
    w = GPT2_WIDTH
    specs = [TensorSpec("wte", (VOCAB, w), True), TensorSpec("wpe", (1024, w), True)]
    for layer in range(GPT2_LAYERS):
        for nm, n in (("ln_1.weight", w), ("ln_1.bias", w), ("attn.c_attn.bias", 3 * w), ("attn.c_proj.bias", w),
                      ("ln_2.weight", w), ("ln_2.bias", w), ("mlp.c_fc.bias", 4 * w), ("mlp.c_proj.bias", w)):
            specs.append(TensorSpec(f"h.{layer}.{nm}", (n,), False))
    specs += [TensorSpec("ln_f.weight", (w,), False), TensorSpec("ln_f.bias", (w,), False)]
    return specs


def make_adamw_tensor(idx: int, spec: TensorSpec, step: int = 1, moments: bool = False) -> dict:
    """Inputs for one AdamW tensor: params, a gradient for `step`, and the
    moments (zero, or drawn when `moments`)."""
    rng = _rng(ADAMW_SEED, idx, 0)
    p = rng.standard_normal(spec.shape, dtype=np.float32) * np.float32(0.02)
    scale = 1e-3 * 10.0 ** _rng(ADAMW_SEED, idx, 1 << 20).uniform(-1.0, 1.0)
    g = _rng(ADAMW_SEED, idx, step).standard_normal(spec.shape, dtype=np.float32) * np.float32(scale)
    if moments:
        mr = _rng(ADAMW_SEED, idx, 1 << 21)
        u = mr.standard_normal(spec.shape, dtype=np.float32) * np.float32(1e-3)
        v = np.square(mr.standard_normal(spec.shape, dtype=np.float32) * np.float32(1e-3))
    else:
        u = np.zeros(spec.shape, np.float32)
        v = np.zeros(spec.shape, np.float32)
    return {"spec": spec, "p": p, "g": g, "u": u, "v": v}
