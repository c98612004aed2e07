"""The layer entry points against the CPU oracle.

Bar: per-row relative Frobenius error of Y <= 5e-3 on every checked row; a row
whose reference is zero must come out exactly zero; no non-finite output.
Small and ragged shapes are checked on every row; so is the sparse + LoRA
layer at every full-size workload, in the same launch configuration the
benchmark times (its dense comparison layer there on sampled rows spanning
first/last tiles, tile boundaries and the interior).
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, sample_rows, say
from workloads import CONFIGS, bf16_bits_from_f32, make_activation, make_layer, make_weights

pytestmark = pytest.mark.gpu


def check(Yg, Yref, label):
    Yg = host_f64(Yg)
    rep = report(label, Yg, Yref)
    zero = np.linalg.norm(Yref, axis=1) == 0
    assert np.all(Yg[zero] == 0), f"{label}: zero rows"
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL, label


# Problems under 16 output tiles of 256 x 256 run the 64 x 64 kernels, larger
# ones the tiled kernels: both families, with ragged M and N tails (N % 8 != 0
# takes the element-wise store path).
SHAPES = [
    (256, 512, 512, 64),     # the tiny workload
    (1, 128, 1, 16), (17, 256, 40, 32), (100, 640, 130, 48), (300, 1152, 257, 64),
    (64, 128, 64, 0), (513, 384, 520, 64), (37, 2048, 300, 16),
    (1000, 640, 1100, 64), (777, 1152, 1030, 48), (520, 256, 1288, 16), (1024, 512, 1024, 0),
    (1280, 3072, 768, 32), (1024, 128, 1024, 64), (1024, 384, 1100, 32),
]


@pytest.mark.parametrize("M,K,N,R", SHAPES)
def test_linear_sparse_lora_shapes(M, K, N, R):
    L = make_layer(M, K, N, "heavy", seed=M + N, R=max(R, 16))
    LA, LB = (None, None) if R == 0 else (L.LA, L.LB)
    say(f"linear_sparse_lora M={M} K={K} N={N} R={R}")
    Y = gu.sparse_lora(dev(L.X), dev(L.W), None if R == 0 else dev(LA),
                                None if R == 0 else dev(LB))
    torch.cuda.synchronize()
    check(Y, orc.linear_sparse_lora(L.X, L.W, LA, LB), f"sparse_lora {M}x{K}->{N} R{R}")


def test_ragged_wide_tiles_sampled_rows():
    """Several rounds of 256-wide tiles (the width the launcher keeps when 192
    would not save a round) with ragged M and N tails; the smaller tiled
    shapes above run 192-wide tiles."""
    M, K, N, R = 4046, 640, 12188, 48
    L = make_layer(M, K, N, "heavy", seed=5, R=R)
    rows = np.unique(np.concatenate([sample_rows(M, n=24, seed=5), np.arange(M - 40, M)]))
    say(f"ragged wide tiles M={M} K={K} N={N} R={R}")
    Y = gu.sparse_lora(dev(L.X), dev(L.W), dev(L.LA), dev(L.LB))
    Yd = gu.dense(dev(L.X), dev(L.W))
    torch.cuda.synchronize()
    check(torch.from_numpy(host_f64(Y)[rows]), orc.linear_sparse_lora(L.X[rows], L.W, L.LA, L.LB),
          "ragged wide sparse_lora")
    check(torch.from_numpy(host_f64(Yd)[rows]), orc.linear_dense(L.X[rows], L.W), "ragged wide dense")


@pytest.mark.parametrize("M,K,N,R", SHAPES[:5] + SHAPES[8:10])
def test_linear_packed_entry(M, K, N, R):
    """The GEMM half on the oracle's own packed operand."""
    L = make_layer(M, K, N, "gelu", seed=M + 3, R=max(R, 16))
    ref = orc.sparsify(L.X, L.LB)
    T_bits = bf16_bits_from_f32(ref.T.astype(np.float32))
    scale = torch.from_numpy(ref.scale.astype(np.float32)).cuda()
    meta = torch.from_numpy(ref.meta_stored()).cuda()
    say(f"packed M={M} K={K} N={N} R={R}")
    Y = gu.packed(dev(ref.values_stored()), meta, scale, dev(T_bits),
                                       dev(L.W), dev(L.LA))
    torch.cuda.synchronize()
    Yref = orc.linear_from_packed(ref.values, ref.meta, ref.scale.astype(np.float32), T_bits,
                                  L.W, L.LA, K)
    check(Y, Yref, f"packed {M}x{K}->{N}")


@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (1, 128, 1), (17, 256, 40), (300, 1152, 257),
                                   (513, 384, 520), (1000, 640, 1100), (520, 256, 1288),
                                   (1024, 1024, 1030)])
def test_linear_dense_shapes(M, K, N):
    L = make_layer(M, K, N, "heavy", seed=M + K + N, R=16)
    say(f"dense M={M} K={K} N={N}")
    Y = gu.dense(dev(L.X), dev(L.W))
    torch.cuda.synchronize()
    check(Y, orc.linear_dense(L.X, L.W), f"dense {M}x{K}->{N}")


def test_identity_two_sparse_input_without_lora_is_dense():
    """Input with <= 2 nonzeros per group and LA = 0: the layer is X W^T."""
    rng = np.random.default_rng(4)
    M, K, N = 200, 768, 300
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = x.reshape(M, K // 4, 4)
    drop = np.argsort(rng.random((M, K // 4, 4)), axis=-1)[..., :2]
    np.put_along_axis(g, drop, 0.0, axis=-1)
    Xb = bf16_bits_from_f32(x)
    W, LA, LB = make_weights(N, K, 64, seed=4)
    say("identity: 2-sparse input, LA = 0")
    Y = gu.sparse_lora(dev(Xb), dev(W), dev(np.zeros_like(LA)), dev(LB))
    Yd = gu.dense(dev(Xb), dev(W))
    torch.cuda.synchronize()
    check(Y, orc.linear_dense(Xb, W), "identity vs oracle dense")
    assert torch.equal(Y.view(torch.int16), Yd.view(torch.int16)) or \
        np.max(np.abs(host_f64(Y) - host_f64(Yd))) <= 2.0 ** -7 * np.abs(host_f64(Yd)).max()


def test_identity_zero_weight_leaves_lora():
    L = make_layer(130, 512, 96, "heavy", seed=5)
    say("identity: W = 0")
    Y = gu.sparse_lora(dev(L.X), dev(np.zeros_like(L.W)), dev(L.LA), dev(L.LB))
    torch.cuda.synchronize()
    Yref = (orc.decode_bf16(L.X) @ orc.decode_bf16(L.LB).T) @ orc.decode_bf16(L.LA).T
    check(Y, Yref, "W = 0")


def test_plus_minus_one_input_scale_sqrt2():
    rng = np.random.default_rng(6)
    M, K, N = 64, 256, 128
    Xb = np.where(rng.random((M, K)) < 0.5, 0x3F80, 0xBF80).astype(np.uint16)
    W, LA, LB = make_weights(N, K, 64, seed=6)
    say("+-1 input")
    Y = gu.sparse_lora(dev(Xb), dev(W), dev(LA), dev(LB))
    torch.cuda.synchronize()
    check(Y, orc.linear_sparse_lora(Xb, W, LA, LB), "+-1 input")


def full_size_layers():
    out = []
    for cfg in ("qkv", "mlp_up", "mlp_down", "block"):
        for i, (M, K, N, kind) in enumerate(CONFIGS[cfg]):
            out.append((cfg, i))
    return out


@pytest.mark.parametrize("cfg,layer", full_size_layers())
def test_full_size_layers(cfg, layer):
    """Every output row of the sparse + LoRA layer against the oracle; the
    dense layer on sampled rows."""
    M, K, N, kind = CONFIGS[cfg][layer]
    L = make_layer(M, K, N, kind, seed=layer)
    rows = sample_rows(M, n=24, seed=layer)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    say(f"full {cfg}[{layer}] M={M} K={K} N={N}")
    Y = gu.sparse_lora(X, W, LA, LB)
    Yd = gu.dense(X, W)
    torch.cuda.synchronize()
    Yh = host_f64(Y)
    Ydh = host_f64(Yd)[rows]
    del X, W, LA, LB, Y, Yd
    say(f"full {cfg}[{layer}]: oracle on all {M} rows")
    check(torch.from_numpy(Yh), orc.linear_sparse_lora(L.X, L.W, L.LA, L.LB),
          f"{cfg}[{layer}] sparse_lora, all rows")
    check(torch.from_numpy(Ydh), orc.linear_dense(L.X[rows], L.W), f"{cfg}[{layer}] dense")
