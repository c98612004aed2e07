"""Seeded generators for the DiT-shaped workloads of the RT-Lynx linear layer.

The RT-Lynx page (aitrends.kr, "RT-Lynx: Diffusion Transformers에서 GEMM
Sparsity를 Activation으로 옮겨 실현하는 방법", section 기술 상세) applies the
sparse linear to the QKV projections and the MLP up/down projections of DiT
blocks.  Real DiT activations and weights are not available, so every input
here is synthetic, with the shapes and value distributions listed in CONFIGS:

* heavy-tailed activations (QKV, attention-out, MLP-up inputs):
  x[m, k] = Laplace(0, 1) * c[k], c[k] ~ LogNormal(0, 1), and the first
  round(1% of K) channels of a seeded permutation get c[k] *= 20 (outliers);
* post-GELU activations (MLP-down inputs):
  x[m, k] = GELU(z[m, k]) * c[k], z ~ N(0, 1), exact erf GELU, c ~ LogNormal(0, 1);
* W ~ N(0, 1/K), LA ~ N(0, 0.02^2), LB ~ N(0, 0.02^2).

All values are drawn in fp32 (fp64 where numpy offers nothing else) and
rounded to bf16 with round-to-nearest-even.  Arrays of bf16 are carried as
their uint16 bit patterns.  Random streams come from numpy's PCG64 seeded
through SeedSequence(seed).spawn, one independent stream per tensor.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf

R_LORA = 64

# name -> list of layers (M, K, N, activation kind); one layer except the block.
CONFIGS: dict[str, list[tuple[int, int, int, str]]] = {
    # tiny correctness case: X [256 x 512], W [512 x 512]
    "tiny": [(256, 512, 512, "heavy")],
    # joint-attention QKV projection of a 1024x1024 latent, 64x64 patch tokens
    "qkv": [(4096, 3072, 9216, "heavy")],
    # MLP up-projection
    "mlp_up": [(4096, 3072, 12288, "heavy")],
    # MLP down-projection, post-GELU input
    "mlp_down": [(4096, 12288, 3072, "gelu")],
    # CFG-batched block: 2 x (4096 image + 512 text) tokens, four linears in order
    "block": [
        (9216, 3072, 9216, "heavy"),
        (9216, 3072, 3072, "heavy"),
        (9216, 3072, 12288, "heavy"),
        (9216, 12288, 3072, "gelu"),
    ],
}
BLOCK_LAYER_NAMES = ("qkv", "attn_out", "mlp_up", "mlp_down")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite by construction; NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, n: int) -> list[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _channel_scales(rng_c: np.random.Generator, rng_o: np.random.Generator, K: int,
                    outliers: bool) -> np.ndarray:
    c = rng_c.lognormal(mean=0.0, sigma=1.0, size=K)
    if outliers:
        n_out = int(round(0.01 * K))
        c[rng_o.permutation(K)[:n_out]] *= 20.0
    return c.astype(np.float32)


def make_activation(kind: str, M: int, K: int, seed: int) -> np.ndarray:
    """Activation matrix X [M x K] as bf16 bits, one of the two distributions."""
    rng_c, rng_o, rng_x = _streams(seed, 3)
    if kind == "heavy":
        c = _channel_scales(rng_c, rng_o, K, outliers=True)
        x = np.empty((M, K), dtype=np.float32)
        step = max(1, (1 << 22) // K)
        for r0 in range(0, M, step):
            r1 = min(M, r0 + step)
            x[r0:r1] = rng_x.laplace(0.0, 1.0, size=(r1 - r0, K)).astype(np.float32) * c
    elif kind == "gelu":
        c = _channel_scales(rng_c, rng_o, K, outliers=False)
        x = np.empty((M, K), dtype=np.float32)
        step = max(1, (1 << 22) // K)
        for r0 in range(0, M, step):
            r1 = min(M, r0 + step)
            z = rng_x.standard_normal(size=(r1 - r0, K))
            g = 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))
            x[r0:r1] = g.astype(np.float32) * c
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    return bf16_bits_from_f32(x)


def make_weights(N: int, K: int, R: int, seed: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """W [N x K] ~ N(0, 1/K); LA [N x R], LB [R x K] ~ N(0, 0.02^2); bf16 bits."""
    rng_w, rng_a, rng_b = _streams(seed + 1_000_003, 3)
    W = rng_w.standard_normal(size=(N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    LA = rng_a.standard_normal(size=(N, R), dtype=np.float32) * np.float32(0.02)
    LB = rng_b.standard_normal(size=(R, K), dtype=np.float32) * np.float32(0.02)
    return bf16_bits_from_f32(W), bf16_bits_from_f32(LA), bf16_bits_from_f32(LB)


@dataclass
class LayerInputs:
    name: str
    M: int
    K: int
    N: int
    R: int
    kind: str
    seed: int
    X: np.ndarray = field(repr=False)
    W: np.ndarray = field(repr=False)
    LA: np.ndarray = field(repr=False)
    LB: np.ndarray = field(repr=False)

    @property
    def dense_equiv_flops(self) -> int:
        """2MNK of the main product plus 2MR(K+N) of the LoRA branch."""
        return 2 * self.M * self.N * self.K + 2 * self.M * self.R * (self.K + self.N)


def make_layer(M: int, K: int, N: int, kind: str = "heavy", seed: int = 0, R: int = R_LORA,
               name: str = "custom") -> LayerInputs:
    X = make_activation(kind, M, K, seed)
    W, LA, LB = make_weights(N, K, R, seed)
    return LayerInputs(name, M, K, N, R, kind, seed, X, W, LA, LB)


def make_config(config: str, seed: int = 0) -> list[LayerInputs]:
    """All layers of a named workload; the block's layers use seeds seed+0..3."""
    layers = CONFIGS[config]
    out = []
    for i, (M, K, N, kind) in enumerate(layers):
        name = config if len(layers) == 1 else f"{config}.{BLOCK_LAYER_NAMES[i]}"
        out.append(make_layer(M, K, N, kind, seed + i, R_LORA, name))
    return out
