"""K a multiple of 64 but not of 128, and K = 64, against the oracle.

With K % 128 == 64 the sparsifier's last 128-channel chunk is 64 channels wide
(the lanes of its upper half load nothing and store nothing) and the tiled
sparse GEMM runs an odd number of 64-channel stages through its LDS ring;
K = 64 runs the 64 x 64 kernels whatever the tile count.  Shapes cover the
sparsifier's 1-, 2- and 3-row-tile workgroups (M = 300, 5000, 9000), a row
that takes the exact fp64 norm pass, the tiled GEMMs with 3, 5 and 7 stages
(192- and 256-wide tiles, ragged tails) and the 64 x 64 kernels.

Bars as in the other parity tests: packed values and meta bit-exact, s within
1e-5 relative, T and Y within 5e-3 per-row relative Frobenius error.
"""
import numpy as np
import pytest
import torch

import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import dev, say
from tests.test_gpu_linear import check
from tests.test_gpu_sparsify import check_sparsify
from workloads import make_activation, make_layer, make_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,R", [(1, 64, 16), (37, 64, 64), (300, 192, 64), (100, 320, 48),
                                   (48, 576, 0), (5000, 192, 64), (9000, 320, 32)])
def test_sparsify_k_multiple_of_64(M, K, R):
    Xb = make_activation("heavy", M, K, seed=M + K)
    if M >= 300:
        Xb[M // 2] = 0x7F7F   # squares overflow fp32: the exact pass
    LB = None if R == 0 else make_weights(8, K, R, seed=R)[2]
    check_sparsify(Xb, LB, f"K%64 {M}x{K} R{R}")


@pytest.mark.parametrize("M,K,N,R", [
    (256, 64, 512, 64),      # 64 x 64 kernels (2 tiles)
    (1024, 64, 1024, 64),    # 16 tiles, but K = 64: 64 x 64 kernels
    (1024, 192, 1024, 64),   # tiled, 3 stages
    (1000, 320, 1100, 48),   # tiled, 5 stages, ragged M and N
    (2048, 448, 2304, 16),   # tiled, 7 stages
])
def test_layer_and_dense_k_multiple_of_64(M, K, N, R):
    L = make_layer(M, K, N, "heavy", seed=M + K, R=R)
    say(f"K%64 layer M={M} K={K} N={N} R={R}")
    X, W = dev(L.X), dev(L.W)
    Y = gu.sparse_lora(X, W, dev(L.LA), dev(L.LB))
    Yd = gu.dense(X, W)
    torch.cuda.synchronize()
    check(Y, orc.linear_sparse_lora(L.X, L.W, L.LA, L.LB), f"sparse_lora {M}x{K}->{N} R{R}")
    check(Yd, orc.linear_dense(L.X, L.W), f"dense {M}x{K}->{N}")
