"""Seeded random shapes through the sparsifier and both layer entry points,
against the CPU oracle.

The shapes are drawn once from a fixed seed, so the set is the same on every
run:
- M and N anywhere from 1 to a few thousand, ragged against the 16-row operand
  tiles, the 64- and 256-row output tiles and the 8-column store vectors;
- K any multiple of 64 up to 2048, so odd stage counts and 64-wide last
  sparsifier chunks are included;
- R in {0, 16, 32, 48, 64};
- heavy-tailed or post-GELU activations.
Even draws have at least 16 output tiles of 256 x 256 and K >= 128, so they run
the tiled kernels. Odd draws are smaller and run the 64 x 64 kernels.

Bars, every row: selection and packed operand bit-exact; s within 1e-5
relative; T and Y within 5e-3 per-row relative error (the dense layer too).
"""
import numpy as np
import pytest

import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import dev, say
from tests.test_gpu_linear import check
from tests.test_gpu_sparsify import check_sparsify
from workloads import make_layer

N_CASES = 16


def draw_shapes(n: int = N_CASES, seed: int = 2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 2 == 0:  # tiled kernels: >= 16 tiles of 256 x 256, K >= 128
            M, N = int(rng.integers(1024, 2900)), int(rng.integers(1024, 2600))
            K = 64 * int(rng.integers(2, 33))
        else:           # 64 x 64 kernels
            M, N = int(rng.integers(1, 700)), int(rng.integers(1, 900))
            K = 64 * int(rng.integers(1, 33))
        R = int(rng.choice([0, 16, 32, 48, 64]))
        kind = "heavy" if rng.random() < 0.5 else "gelu"
        out.append((M, K, N, R, kind))
    return out


SWEEP = draw_shapes()


def test_sweep_spans_both_kernel_families():
    """The draw covers both kernel families, odd stage counts, no LoRA and
    rank 64, and ragged M and N."""
    tiled = [(M, K, N) for M, K, N, _, _ in SWEEP
             if -(-M // 256) * -(-N // 256) >= 16 and K >= 128]
    assert len(tiled) == N_CASES // 2
    assert any(K % 128 == 64 for _, K, _, _, _ in SWEEP)
    assert {R for *_, R, _ in SWEEP} >= {0, 64}
    assert any(M % 16 for M, *_ in SWEEP) and any(N % 8 for _, _, N, _, _ in SWEEP)


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,R,kind", SWEEP)
def test_random_shape(M, K, N, R, kind):
    L = make_layer(M, K, N, kind, seed=M * 7 + N, R=max(R, 16))
    LA, LB = (None, None) if R == 0 else (L.LA, L.LB)
    label = f"{kind} {M}x{K}->{N} R{R}"
    check_sparsify(L.X, LB, label)
    say(f"sweep layers {label}")
    Ys = gu.sparse_lora(dev(L.X), dev(L.W), None if R == 0 else dev(LA), None if R == 0 else dev(LB))
    Yd = gu.dense(dev(L.X), dev(L.W))
    check(Ys, orc.linear_sparse_lora(L.X, L.W, LA, LB), f"sweep sparse_lora {label}")
    check(Yd, orc.linear_dense(L.X, L.W), f"sweep dense {label}")
