"""The method's edge cases through the tiled kernels every workload runs.

Problems of at least 16 output tiles of 256 x 256 run the persistent tiled
GEMMs; these tests take the layer's identities and its norm-compensation
extremes through them, at 1024 x 512 -> 1024 (16 tiles) and at the MLP-up
shape 4096 x 3072 -> 12288:

* rows of +-1 (every group tied, s = sqrt 2), rows with at most two nonzeros
  per group (s = 1) and heavy-tailed rows interleaved, so every 32-row
  accumulator block holds s spanning [1, sqrt 2], with a LoRA branch of the
  same order as the sparse product: the page's second formula (코드 예제)
  scales only S(X) W^T, and each test also asserts that the alternative
  s (X~ W^T + T LA^T) misses the oracle by far more than the tolerance;
* W = 0, where the layer is (X LB^T) LA^T;
* LA = 0 with input of at most two nonzeros per group, where the layer is
  the dense product X W^T (also compared with the dense kernel);
* no store lands past the end of Y when the last row tile is partial.

Bar: per-row relative Frobenius error <= 5e-3 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, row_rel_err, sample_rows, say
from workloads import bf16_bits_from_f32, make_activation, make_layer, make_weights

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 512, 1024), (4096, 3072, 12288)]


def check(Yg, Yref, label):
    rep = report(label, Yg, Yref)
    zero = np.linalg.norm(Yref, axis=1) == 0
    assert np.all(Yg[zero] == 0), f"{label}: zero rows"
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL, label


def lora_weights(N, K, R, sigma, seed):
    """LA [N x R], LB [R x K] ~ N(0, sigma^2): a LoRA branch comparable to the
    sparse product (the workloads' 0.02 makes it a few percent of it)."""
    rng = np.random.default_rng(seed)
    LA = bf16_bits_from_f32((rng.standard_normal((N, R)) * sigma).astype(np.float32))
    LB = bf16_bits_from_f32((rng.standard_normal((R, K)) * sigma).astype(np.float32))
    return LA, LB


def two_sparse(x, rng):
    """Zero two random positions of every group of 4 (s = 1 for such rows)."""
    M, K = x.shape
    g = x.reshape(M, K // 4, 4)
    drop = np.argsort(rng.random((M, K // 4, 4)), axis=-1)[..., :2]
    np.put_along_axis(g, drop, 0.0, axis=-1)
    return g.reshape(M, K)


def mixed_rows(M, K, seed):
    """Row m % 3 == 0: +-1; == 1: Gaussian with two zeros per group; == 2:
    the heavy-tailed workload distribution."""
    rng = np.random.default_rng(seed)
    Xb = make_activation("heavy", M, K, seed=seed)
    pm = np.where(rng.random((M, K)) < 0.5, 0x3F80, 0xBF80).astype(np.uint16)
    sp = bf16_bits_from_f32(two_sparse(rng.standard_normal((M, K)).astype(np.float32), rng))
    kind = np.arange(M) % 3
    Xb[kind == 0] = pm[kind == 0]
    Xb[kind == 1] = sp[kind == 1]
    return Xb


def checked_rows(M):
    """All rows of a small problem; three whole 256-row tiles (first, middle,
    last) plus sampled rows of a large one."""
    if M <= 1024:
        return np.arange(M)
    mid = (M // 512) * 256
    return np.unique(np.concatenate([np.arange(256), np.arange(mid, mid + 256),
                                     np.arange(M - 256, M), sample_rows(M, n=32, seed=M)]))


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_scale_spanning_one_to_sqrt2_with_lora(M, K, N):
    Xb = mixed_rows(M, K, seed=11)
    W = make_weights(N, K, 16, seed=12)[0]
    LA, LB = lora_weights(N, K, 64, 0.05, seed=13)
    rows = checked_rows(M)
    say(f"edges: s in [1, sqrt2] with LoRA M={M} K={K} N={N}")
    Y = gu.sparse_lora(dev(Xb), dev(W), dev(LA), dev(LB))
    torch.cuda.synchronize()
    Yg = host_f64(Y)[rows]
    del Y
    ref = orc.sparsify(Xb[rows], LB)
    kinds = rows % 3
    assert np.allclose(ref.scale[kinds == 0], np.sqrt(2), rtol=1e-15)
    assert np.all(ref.scale[kinds == 1] == 1.0)
    Yref = orc.linear_sparse_lora(Xb[rows], W, LA, LB)
    check(Yg, Yref, f"s in [1, sqrt2] {M}x{K}->{N}")
    # the order the page fixes is what this test tells apart: s applied after
    # the LoRA term would miss the oracle by >= 10x the tolerance on the
    # +-1 rows
    Yr = ref.T @ orc.decode_bf16(LA).T
    wrong = Yref + (ref.scale[:, None] - 1.0) * Yr
    assert row_rel_err(wrong[kinds == 0], Yref[kinds == 0]).min() > 10 * ROW_REL_TOL
    assert row_rel_err(Yg[kinds == 0], wrong[kinds == 0]).min() > 5 * ROW_REL_TOL


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_zero_weight_leaves_lora(M, K, N):
    Xb = mixed_rows(M, K, seed=21)
    LA, LB = lora_weights(N, K, 64, 0.05, seed=22)
    W0 = np.zeros((N, K), dtype=np.uint16)
    rows = checked_rows(M)
    say(f"edges: W = 0 M={M} K={K} N={N}")
    Y = gu.sparse_lora(dev(Xb), dev(W0), dev(LA), dev(LB))
    torch.cuda.synchronize()
    Yg = host_f64(Y)[rows]
    del Y
    x = orc.decode_bf16(Xb[rows])
    Yref = (x @ orc.decode_bf16(LB).T) @ orc.decode_bf16(LA).T
    check(Yg, Yref, f"W = 0 {M}x{K}->{N}")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_two_sparse_input_without_lora_is_dense(M, K, N):
    rng = np.random.default_rng(31)
    Xb = bf16_bits_from_f32(two_sparse(
        (rng.laplace(size=(M, K)) * np.exp(rng.standard_normal(K))).astype(np.float32), rng))
    W, LA, LB = make_weights(N, K, 64, seed=32)
    LA0 = np.zeros_like(LA)
    rows = checked_rows(M)
    say(f"edges: 2-sparse input, LA = 0 M={M} K={K} N={N}")
    Xd, Wd = dev(Xb), dev(W)
    Y = gu.sparse_lora(Xd, Wd, dev(LA0), dev(LB))
    Yd = gu.dense(Xd, Wd)
    torch.cuda.synchronize()
    Yg, Ydg = host_f64(Y), host_f64(Yd)
    del Xd, Wd, Y, Yd
    ref = orc.linear_dense(Xb[rows], W)
    check(Yg[rows], ref, f"2-sparse, LA = 0 {M}x{K}->{N}")
    check(Ydg[rows], ref, f"2-sparse dense kernel {M}x{K}->{N}")
    # both kernels sum the same products in fp32: they agree to a few bf16 ulps
    assert row_rel_err(Yg, Ydg).max() <= ROW_REL_TOL


SENTINEL = 0x7E57  # a bf16 NaN pattern no kernel produces from finite inputs


@pytest.mark.parametrize("M,K,N,R", [(520, 256, 1288, 16), (4100, 512, 1024, 64),
                                     (4046, 128, 12288, 32)])
def test_no_store_past_the_end_of_Y(M, K, N, R):
    """Ragged M (the last row tile partial) with N % 8 == 0, so interior tiles
    store straight from the accumulators: Y is the head of a larger buffer
    whose tail must come back untouched, for both GEMMs (192- and 256-wide
    tiles)."""
    L = make_layer(M, K, N, "heavy", seed=M + 1, R=R)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    tail = 256 * N + 64
    rows = np.unique(np.concatenate([np.arange(M - 48, M), sample_rows(M, n=16, seed=M)]))
    for which in ("sparse", "dense"):
        buf = torch.full((M * N + tail,), SENTINEL, dtype=torch.int16, device="cuda")
        Y = buf[:M * N].view(torch.bfloat16).view(M, N)
        say(f"edges: no store past Y ({which}) M={M} K={K} N={N} R={R}")
        if which == "sparse":
            lynx.linear_sparse_lora(X, W, LA, LB, Y=Y)
        else:
            lynx.linear_dense(X, W, Y=Y)
        torch.cuda.synchronize()
        tail_bits = buf[M * N:].cpu().numpy()
        assert np.all(tail_bits == SENTINEL), \
            f"{which}: {int(np.sum(tail_bits != SENTINEL))} stores past the end of Y"
        Yg = host_f64(Y)[rows]
        ref = (orc.linear_sparse_lora(L.X[rows], L.W, L.LA, L.LB) if which == "sparse"
               else orc.linear_dense(L.X[rows], L.W))
        check(Yg, ref, f"{which} {M}x{K}->{N} rows near the end")
        del buf, Y
