"""lynx_sparsify (K1) against the CPU oracle.

Bar: selected indices (through meta) and kept values bit-exact; scale within
1e-5 relative; T within 5e-3 per-row relative error.  Shapes cover several
row blocks with ragged tails, every supported rank, adversarial groups (ties,
zeros, -0, +-1, denormals, extremes) and the full-size workloads.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import (ROW_REL_TOL, SCALE_REL_TOL, dev, host_bits, host_f64, report,
                            row_rel_err, say)
from workloads import CONFIGS, make_activation, make_weights

pytestmark = pytest.mark.gpu


def check_sparsify(Xb, LBb, label):
    """Stored packed operand (incl. padding rows) bit-exact, scale, T."""
    M, K = Xb.shape
    say(f"sparsify {label} M={M} K={K} R={0 if LBb is None else LBb.shape[0]}")
    values, meta, scale, T = gu.sparsify(dev(Xb), None if LBb is None else dev(LBb))
    torch.cuda.synchronize()
    ref = orc.sparsify(Xb, LBb)
    np.testing.assert_array_equal(meta.cpu().numpy(), ref.meta_stored(), err_msg=f"{label}: meta")
    np.testing.assert_array_equal(host_bits(values), ref.values_stored(),
                                  err_msg=f"{label}: values")
    s = scale.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(s / ref.scale - 1)) <= SCALE_REL_TOL, f"{label}: scale"
    if LBb is not None:
        Tg = host_f64(T)
        rep = report(f"{label} T", Tg, ref.T)
        zero = np.linalg.norm(ref.T, axis=1) == 0
        assert np.all(Tg[zero] == 0)
        assert rep["max_row_rel"] <= ROW_REL_TOL and rep["nonfinite"] == 0


@pytest.mark.parametrize("M,K,R", [
    (256, 512, 64),    # the tiny workload
    (1, 128, 16), (17, 256, 32), (100, 640, 48), (33, 1152, 64), (16, 128, 0), (255, 1024, 64),
])
def test_sparsify_shapes(M, K, R):
    Xb = make_activation("heavy", M, K, seed=M + K)
    LB = None if R == 0 else make_weights(8, K, R, seed=R)[2]
    check_sparsify(Xb, LB, f"heavy {M}x{K}")


@pytest.mark.parametrize("M,R", [(5000, 64), (4120, 48), (8192, 64), (9000, 64), (12000, 16)])
def test_sparsify_many_row_blocks(M, R):
    """More 16-row tiles than compute units, so workgroups take 2 (M = 4120,
    5000, 8192) or 3 (M = 9000, 12000) row tiles each, with ragged and exact M:
    the last workgroup of M = 9000 holds a partial tile and a tile past the
    padded rows, which it must not write (a write past the packed buffers
    lands in the next output and shows up as a wrong scale)."""
    Xb = make_activation("heavy", M, 384, seed=M)
    check_sparsify(Xb, make_weights(8, 384, R, seed=R)[2], f"heavy {M}x384")


@pytest.mark.parametrize("M,K,R", [(9000, 128, 64), (5000, 256, 32), (12000, 128, 16)])
def test_sparsify_row_tiles_few_waves(M, K, R):
    """Workgroups of 2 or 3 row tiles whose K has only one or two 128-channel
    chunks, so they run with fewer waves than rows to reduce."""
    Xb = make_activation("heavy", M, K, seed=M + K)
    check_sparsify(Xb, make_weights(8, K, R, seed=R)[2], f"heavy {M}x{K} R{R}")


def test_sparsify_gelu_input():
    Xb = make_activation("gelu", 64, 3072, seed=3)
    check_sparsify(Xb, make_weights(8, 3072, 64, seed=3)[2], "gelu 64x3072")


def adversarial_rows(specials, M, K, seed):
    rng = np.random.default_rng(seed)
    Xb = specials[rng.integers(0, len(specials), size=(M, K))]
    Xb[0] = 0                                   # zero row
    Xb[1] = 0x8000                              # negative zeros
    Xb[2] = np.where(rng.random(K) < 0.5, 0x3F80, 0xBF80)  # +-1: all ties, s = sqrt(2)
    Xb[3, :] = 0x3F80                           # all equal
    Xb[4] = 0                                   # one nonzero per group
    Xb[4, ::4] = 0x4000
    Xb[5] = rng.choice(np.array([0x0001, 0x8001, 0x0003, 0x007F], dtype=np.uint16), size=K)
    return Xb


def test_sparsify_extreme_magnitudes():
    """Largest finite values and subnormals: selection, packing and s (fp64 path)."""
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                         0x3F80, 0xBF80, 0x4000, 0xC000], dtype=np.uint16)
    Xb = adversarial_rows(specials, 48, 512, seed=0)
    Xb[6] = 0x7F7F                              # every square overflows fp32
    Xb[7, :256] = 0x0080                        # smallest normal next to subnormals
    Xb[7, 256:] = 0x0001
    check_sparsify(Xb, None, "extreme magnitudes")


def test_sparsify_adversarial_groups_with_lora():
    """Ties, zeros, -0, +-1 and subnormals with moderate magnitudes, T included."""
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x4780, 0xC780,
                         0x3F80, 0xBF80, 0x4000, 0xC000], dtype=np.uint16)
    Xb = adversarial_rows(specials, 48, 512, seed=1)
    LB = make_weights(8, 512, 64, seed=0)[2]
    check_sparsify(Xb, LB, "adversarial")


def test_sparsify_is_deterministic():
    Xb = make_activation("heavy", 300, 3072, seed=7)
    LB = make_weights(8, 3072, 64, seed=7)[2]
    X, L = dev(Xb), dev(LB)
    a = [t.clone() for t in gu.sparsify(X, L)]
    b = gu.sparsify(X, L)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)


@pytest.mark.parametrize("M,K,kind", sorted({(m, k, kind) for cfg in ("qkv", "mlp_down", "block")
                                             for (m, k, n, kind) in CONFIGS[cfg]}))
def test_sparsify_full_size(M, K, kind):
    """Full-size activations: meta/values/scale on every row, T on sampled rows."""
    Xb = make_activation(kind, M, K, seed=0)
    LB = make_weights(8, K, 64, seed=0)[2]
    say(f"sparsify full {M}x{K} {kind}")
    values, meta, scale, T = gu.sparsify(dev(Xb), dev(LB))
    torch.cuda.synchronize()
    idx = orc.select_top2_of_4(Xb)
    np.testing.assert_array_equal(meta.cpu().numpy(),
                                  orc.tile_rows(orc.pack_meta(idx), K, 0x44).reshape(-1))
    np.testing.assert_array_equal(host_bits(values),
                                  orc.tile_rows(orc.pack_values(Xb, idx), K, 0).reshape(-1))
    s_ref = orc.norm_scale(orc.decode_bf16(Xb), orc.keep_mask(idx))
    s = scale.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(s / s_ref - 1)) <= SCALE_REL_TOL
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    T_ref = orc.decode_bf16(Xb[rows]) @ orc.decode_bf16(LB).T
    assert row_rel_err(host_f64(T)[rows], T_ref).max() <= ROW_REL_TOL


def extreme_row(kind, K, rng):
    """One row whose squares leave fp32's range (or vanish), so its norm
    takes the exact fp64 pass."""
    sign = np.where(rng.random(K) < 0.5, 0x8000, 0).astype(np.uint16)
    if kind == "max":          # the largest finite bf16: squares overflow fp32
        return (0x7F7F | sign).astype(np.uint16)
    if kind == "huge":         # |x| in [2^70, 2^71): squares overflow fp32
        return (0x6280 + rng.integers(0, 128, K) | sign).astype(np.uint16)
    if kind == "subnormal":    # squares underflow to zero in fp32
        return (rng.integers(1, 128, K) | sign).astype(np.uint16)
    if kind == "tiny":         # 2^-70 .. : squares below 2^-60 in sum
        return (0x1C80 + rng.integers(0, 128, K) | sign).astype(np.uint16)
    if kind == "zero":
        return np.zeros(K, dtype=np.uint16)
    if kind == "mixed":        # smallest normals next to subnormals
        r = (rng.integers(1, 128, K) | sign).astype(np.uint16)
        r[::3] = 0x0080 | sign[::3]
        return r
    raise ValueError(kind)


@pytest.mark.parametrize("M", [5000, 9000])
def test_sparsify_extreme_rows_across_row_tiles(M):
    """Rows that take the exact fp64 norm pass, scattered over row tiles and
    workgroups when a workgroup holds 2 (M = 5000) or 3 (M = 9000) row tiles,
    with the rank-64 LoRA: packed operand bit-exact, s within 1e-5 (and,
    on the exact rows, the fp64 value rounded once to fp32), T on the rows
    whose products stay in range."""
    K, R = 384, 64
    rng = np.random.default_rng(M)
    Xb = make_activation("heavy", M, K, seed=M + 1)
    LB = make_weights(8, K, R, seed=3)[2]
    tiles = (M + 15) // 16
    kinds = ["max", "huge", "subnormal", "tiny", "zero", "mixed"]
    special = {}
    for t in sorted({0, 1, 2, 3, 5, tiles // 3, tiles // 2, tiles - 3, tiles - 2, tiles - 1}):
        for j, r in enumerate((0, 5, 15) if t % 2 == 0 else (3, 8, 12)):
            m = 16 * t + r
            if m < M:
                k = kinds[(t + j) % len(kinds)]
                Xb[m] = extreme_row(k, K, rng)
                special[m] = k
    rows = np.array(sorted(special))
    say(f"sparsify extreme rows M={M} K={K} R={R}: {len(rows)} special rows")
    values, meta, scale, T = gu.sparsify(dev(Xb), dev(LB))
    torch.cuda.synchronize()
    ref = orc.sparsify(Xb, LB)
    np.testing.assert_array_equal(meta.cpu().numpy(), ref.meta_stored(), err_msg="meta")
    np.testing.assert_array_equal(host_bits(values), ref.values_stored(), err_msg="values")
    s = scale.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(s / ref.scale - 1)) <= SCALE_REL_TOL, "scale"
    assert np.max(np.abs(s[rows] / ref.scale[rows] - 1)) <= 2.0 ** -23, "scale of exact rows"
    assert np.all(s[[m for m in rows if special[m] == "zero"]] == 1.0)
    # T: rows of the largest finite value overflow fp32 and bf16 (outside the
    # contract's range); every other row within 5e-3
    ok = np.array([special.get(m) != "max" for m in range(M)])
    Tg = host_f64(T)
    rep = report(f"extreme rows M={M} T", Tg[ok], ref.T[ok])
    assert rep["max_row_rel"] <= ROW_REL_TOL and rep["nonfinite"] == 0
    assert np.all(Tg[[m for m in rows if special[m] == "zero"]] == 0)


def test_sparsify_is_deterministic_three_row_tiles():
    """Workgroups of three row tiles (M = 9000, R = 64): two calls give the
    same bits in every output."""
    Xb = make_activation("heavy", 9000, 3072, seed=9)
    LB = make_weights(8, 3072, 64, seed=9)[2]
    X, L = dev(Xb), dev(LB)
    say("sparsify determinism M=9000 K=3072 R=64 (3 row tiles per workgroup)")
    a = [t.clone() for t in gu.sparsify(X, L)]
    b = gu.sparsify(X, L)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)
