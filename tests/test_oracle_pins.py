"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against one of: the bf16 format definition, a
hand-worked example (tests/golden), an exact brute force over all 2-of-4
masks in rational arithmetic, a closed form, or an identity that reduces the
layer to a textbook product.  Chosen so that a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule, an inverted scale or a wrong
metadata bit order each fails at least one test.

Method source: the RT-Lynx page (aitrends.kr), 방법론 / 핵심 메커니즘 and the
two formulas of 코드 예제.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import lynx_oracle as orc
from workloads import bf16_bits_from_f32, make_activation, make_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact helpers written here from the bf16 definition (not the oracle's)
# ---------------------------------------------------------------------------
def frac_of_bf16(b: int) -> Fraction:
    b = int(b)
    s = -1 if (b >> 15) & 1 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return s * Fraction(f, 128) * Fraction(1, 2 ** 126)
    return s * (1 + Fraction(f, 128)) * (Fraction(2) ** (e - 127))


def brute_force_pair(group_bits) -> tuple[int, int]:
    """Pair (i<j) keeping the most energy; among equal energies the
    lexicographically smallest pair.  For top-2-by-magnitude with ties to the
    lower index this is the same pair: every maximum-energy pair holds the
    largest magnitudes, and the smallest pair prefers lower indices."""
    a2 = [frac_of_bf16(b) ** 2 for b in group_bits]
    best = None
    for i, j in itertools.combinations(range(4), 2):
        e = a2[i] + a2[j]
        if best is None or e > best[0]:
            best = (e, (i, j))
    return best[1]


def brute_force_layer(Xb, Wb, LAb, LBb):
    """Y by exact rational sums; s = sqrt of an exact ratio, rounded once."""
    M, K = Xb.shape
    N = Wb.shape[0]
    R = LBb.shape[0] if LBb is not None else 0
    X = [[frac_of_bf16(v) for v in row] for row in Xb]
    W = [[frac_of_bf16(v) for v in row] for row in Wb]
    Y = np.zeros((M, N))
    for m in range(M):
        keep = [False] * K
        for g in range(K // 4):
            i, j = brute_force_pair(Xb[m, 4 * g:4 * g + 4])
            keep[4 * g + i] = keep[4 * g + j] = True
        n2 = sum(v * v for v in X[m])
        nt2 = sum(v * v for v, k in zip(X[m], keep) if k)
        s = math.sqrt(n2 / nt2) if nt2 else 1.0
        T = []
        for r in range(R):
            T.append(sum(X[m][k] * frac_of_bf16(LBb[r, k]) for k in range(K)))
        for n in range(N):
            ys = sum(X[m][k] * W[n][k] for k in range(K) if keep[k])
            yr = sum(T[r] * frac_of_bf16(LAb[n, r]) for r in range(R)) if R else 0
            Y[m, n] = s * float(ys) + float(yr)
    return Y


# ---------------------------------------------------------------------------
# bf16 decoding, from the format definition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x3F00, 0.5),
    (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126), (0x8000, -0.0),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0xBF80, -1.0),
])
def test_decode_bf16_known_values(bits, value):
    got = orc.decode_bf16(np.array([bits], dtype=np.uint16))[0]
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


def test_decode_bf16_matches_f32_widening_all_finite():
    # every finite bf16 equals the fp32 whose upper half it is
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 7) & 0xFF) != 0xFF
    b = b[finite]
    f32 = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(orc.decode_bf16(b), f32)


# ---------------------------------------------------------------------------
# selection: exhaustive over magnitude orderings with ties, both signs, -0
# ---------------------------------------------------------------------------
MAGS = [0x0000, 0x3F80, 0x4000, 0x4040]  # 0, 1, 2, 3


def test_select_exhaustive_tie_patterns():
    groups = []
    for mags in itertools.product(MAGS, repeat=4):
        for signs in itertools.product((0, 0x8000), repeat=4):
            groups.append([m | s for m, s in zip(mags, signs)])
    Xb = np.array(groups, dtype=np.uint16).reshape(-1, 4)
    idx = orc.select_top2_of_4(Xb)
    for row, got in zip(groups, idx):
        assert tuple(got[0]) == brute_force_pair(row), row


def test_select_extremes_and_denormals():
    specials = [0x0000, 0x8000, 0x0001, 0x8001, 0x0002, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80]
    groups = [list(g) for g in itertools.product(specials, repeat=4)]
    Xb = np.array(groups, dtype=np.uint16)
    idx = orc.select_top2_of_4(Xb)
    for row, got in zip(groups, idx):
        assert tuple(got[0]) == brute_force_pair(row), row


def test_select_random_rows_vs_brute_force():
    Xb = make_activation("heavy", 8, 64, seed=11)
    idx = orc.select_top2_of_4(Xb)
    for m in range(8):
        for g in range(16):
            assert tuple(idx[m, g]) == brute_force_pair(Xb[m, 4 * g:4 * g + 4])


# ---------------------------------------------------------------------------
# hand-worked golden example
# ---------------------------------------------------------------------------
def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "worked_example_3x8.json")) as f:
        g = json.load(f)
    Xb = np.array(g["X_bits"], dtype=np.uint16)
    W = bf16_bits_from_f32(np.array(g["W"], dtype=np.float32))
    LA = bf16_bits_from_f32(np.array(g["LA"], dtype=np.float32))
    LB = bf16_bits_from_f32(np.array(g["LB"], dtype=np.float32))
    e = g["expected"]
    res = orc.sparsify(Xb, LB)
    np.testing.assert_array_equal(res.idx, np.array(e["idx"]))
    np.testing.assert_array_equal(res.meta, np.array(e["meta"], dtype=np.uint8))
    np.testing.assert_array_equal(res.values, np.array(e["values_bits"], dtype=np.uint16))
    s_exp = np.array([math.sqrt(a / b) if b else 1.0 for a, b in e["scale_squared_num_den"]])
    np.testing.assert_allclose(res.scale, s_exp, rtol=1e-15)
    np.testing.assert_allclose(res.T, np.array(e["T"]), rtol=0, atol=0)
    Y = orc.linear_sparse_lora(Xb, W, LA, LB)
    coeff = np.array(e["Y_sparse_coeff_and_lora"])  # [M, N, 2]
    Y_exp = s_exp[:, None] * coeff[..., 0] + coeff[..., 1]
    np.testing.assert_allclose(Y, Y_exp, rtol=1e-15, atol=0)
    # packed -> dense round trip rebuilds x~ exactly
    xt = orc.unpack_dense(res.values, res.meta, 8)
    x = orc.decode_bf16(Xb)
    np.testing.assert_array_equal(xt, np.where(orc.keep_mask(res.idx), x, 0.0))


# ---------------------------------------------------------------------------
# invariants of norm compensation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["heavy", "gelu"])
def test_norm_preserved_and_scale_bounds(kind):
    Xb = make_activation(kind, 32, 256, seed=3)
    res = orc.sparsify(Xb)
    x = orc.decode_bf16(Xb)
    xt = orc.unpack_dense(res.values, res.meta, 256)
    n = np.linalg.norm(x, axis=1)
    nt = np.linalg.norm(res.scale[:, None] * xt, axis=1)
    np.testing.assert_allclose(nt, n, rtol=1e-12)
    assert np.all(res.scale >= 1.0) and np.all(res.scale <= math.sqrt(2) * (1 + 1e-15))


def test_scale_is_one_iff_at_most_two_nonzeros_per_group():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    g = x.reshape(16, 16, 4)
    for m in range(16):
        for j in range(16):
            drop = rng.choice(4, size=2, replace=False)
            g[m, j, drop] = 0.0
    Xb = bf16_bits_from_f32(x)
    assert np.all(orc.sparsify(Xb).scale == 1.0)
    # one extra nonzero in one group of each row makes s > 1
    Xb2 = Xb.copy()
    for m in range(16):
        grp = Xb2[m, :4]
        zero = np.flatnonzero((grp & 0x7FFF) == 0)[0]
        Xb2[m, zero] = 0x3F80
    assert np.all(orc.sparsify(Xb2).scale > 1.0)


def test_power_of_two_scaling_and_sign_flip_exact():
    Xb = make_activation("heavy", 16, 128, seed=9)
    x = orc.decode_bf16(Xb)
    base = orc.sparsify(Xb)
    for factor in (0.25, 4.0):
        Xs = bf16_bits_from_f32((x * factor).astype(np.float32))
        r = orc.sparsify(Xs)
        np.testing.assert_array_equal(r.idx, base.idx)
        np.testing.assert_allclose(r.scale, base.scale, rtol=1e-15)
    neg = Xb ^ np.uint16(0x8000)
    r = orc.sparsify(neg)
    np.testing.assert_array_equal(r.idx, base.idx)
    np.testing.assert_array_equal(r.values, base.values ^ np.uint16(0x8000))
    np.testing.assert_array_equal(r.scale, base.scale)


def test_zero_row():
    Xb = np.zeros((2, 32), dtype=np.uint16)
    Xb[1, ::3] = 0x8000  # negative zeros
    W, LA, LB = make_weights(8, 32, 4, seed=1)
    res = orc.sparsify(Xb, LB)
    assert np.all(res.idx[..., 0] == 0) and np.all(res.idx[..., 1] == 1)
    assert np.all(res.scale == 1.0)
    assert np.all(orc.linear_sparse_lora(Xb, W, LA, LB) == 0.0)


# ---------------------------------------------------------------------------
# special cases reducing to textbook products (expected values by exact sums)
# ---------------------------------------------------------------------------
def test_two_sparse_input_without_lora_is_dense_gemm():
    rng = np.random.default_rng(21)
    M, K, N = 3, 16, 5
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = x.reshape(M, K // 4, 4)
    for m in range(M):
        for j in range(K // 4):
            g[m, j, rng.choice(4, size=2, replace=False)] = 0.0
    Xb = bf16_bits_from_f32(x)
    W, LA, LB = make_weights(N, K, 2, seed=2)
    LA0 = np.zeros_like(LA)
    Y = orc.linear_sparse_lora(Xb, W, LA0, LB)
    Xf = [[frac_of_bf16(v) for v in r] for r in Xb]
    Wf = [[frac_of_bf16(v) for v in r] for r in W]
    Y_exp = np.array([[float(sum(a * b for a, b in zip(Xf[m], Wf[n]))) for n in range(N)]
                      for m in range(M)])
    np.testing.assert_allclose(Y, Y_exp, rtol=1e-13, atol=1e-300)


def test_zero_weight_leaves_lora_of_dense_x():
    Xb = make_activation("heavy", 3, 16, seed=4)
    W, LA, LB = make_weights(5, 16, 3, seed=4)
    W0 = np.zeros_like(W)
    Y = orc.linear_sparse_lora(Xb, W0, LA, LB)
    assert np.all(orc.sparsify(Xb).scale > 1.0)  # s != 1, so a scaled LoRA would show
    Xf = [[frac_of_bf16(v) for v in r] for r in Xb]
    T = [[sum(Xf[m][k] * frac_of_bf16(LB[r, k]) for k in range(16)) for r in range(3)]
         for m in range(3)]
    Y_exp = np.array([[float(sum(T[m][r] * frac_of_bf16(LA[n, r]) for r in range(3)))
                       for n in range(5)] for m in range(3)])
    np.testing.assert_allclose(Y, Y_exp, rtol=1e-13)


def test_all_plus_minus_one_closed_form():
    rng = np.random.default_rng(8)
    M, K, N = 4, 32, 6
    Xb = np.where(rng.random((M, K)) < 0.5, 0x3F80, 0xBF80).astype(np.uint16)
    W, LA, LB = make_weights(N, K, 4, seed=8)
    res = orc.sparsify(Xb, LB)
    assert np.all(res.idx[..., 0] == 0) and np.all(res.idx[..., 1] == 1)
    np.testing.assert_allclose(res.scale, math.sqrt(2), rtol=1e-15)
    x = orc.decode_bf16(Xb)
    xt = x.copy().reshape(M, K // 4, 4)
    xt[..., 2:] = 0.0
    Y_exp = math.sqrt(2) * (xt.reshape(M, K) @ orc.decode_bf16(W).T) \
        + (x @ orc.decode_bf16(LB).T) @ orc.decode_bf16(LA).T
    np.testing.assert_allclose(orc.linear_sparse_lora(Xb, W, LA, LB), Y_exp, rtol=1e-13)


# ---------------------------------------------------------------------------
# tiny layers: the whole Y against exact brute force
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,R,seed", [(4, 32, 5, 3, 0), (3, 16, 8, 2, 1), (8, 8, 3, 1, 2)])
def test_tiny_layer_brute_force(M, K, N, R, seed):
    Xb = make_activation("heavy", M, K, seed)
    W, LA, LB = make_weights(N, K, R, seed)
    Y = orc.linear_sparse_lora(Xb, W, LA, LB)
    np.testing.assert_allclose(Y, brute_force_layer(Xb, W, LA, LB), rtol=1e-12, atol=1e-12)


def test_packed_path_equals_layer():
    Xb = make_activation("gelu", 6, 64, seed=6)
    W, LA, LB = make_weights(7, 64, 4, seed=6)
    res = orc.sparsify(Xb, LB)
    # with T kept exactly (as fp64 bits cannot be bf16, use a bf16-exact T)
    Y_packed = orc.linear_from_packed(res.values, res.meta, res.scale, None, W, None, 64)
    Y_ref = orc.linear_sparse_lora(Xb, W, np.zeros_like(LA), LB)
    np.testing.assert_allclose(Y_packed, Y_ref, rtol=1e-13)


def test_packed_path_with_lora_brute_force():
    """linear_from_packed with its LoRA term: small-integer X and LB make
    T = X LB^T exactly representable in bf16, so the packed path given the
    packed operand, s and that T must reproduce the whole layer, which is
    summed here by exact rational brute force from X.  The LoRA term is made
    comparable to the sparse term and s > 1 on every row, so a dropped,
    negated, s-scaled or mis-oriented T LA^T term fails."""
    rng = np.random.default_rng(21)
    M, K, N, R = 3, 16, 5, 4
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    x[:, 0::4] = np.where(x[:, 0::4] == 0, 1.0, x[:, 0::4])   # >= 3 nonzeros in every group,
    x[:, 1::4] = np.where(x[:, 1::4] == 0, -2.0, x[:, 1::4])  # so s > 1 on every row
    x[:, 2::4] = np.where(x[:, 2::4] == 0, 3.0, x[:, 2::4])
    Xb = bf16_bits_from_f32(x)
    LB = bf16_bits_from_f32(rng.integers(-1, 2, size=(R, K)).astype(np.float32))
    LA = bf16_bits_from_f32(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(N, R)).astype(np.float32))
    W = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.25).astype(np.float32))
    res = orc.sparsify(Xb, LB)
    assert np.all(res.scale > 1.0)
    T_exact = [[sum(frac_of_bf16(Xb[m, k]) * frac_of_bf16(LB[r, k]) for k in range(K))
                for r in range(R)] for m in range(M)]
    assert all(t.denominator == 1 and abs(t) <= 256 for row in T_exact for t in row)
    T_bits = bf16_bits_from_f32(np.array([[float(t) for t in row] for row in T_exact],
                                         dtype=np.float32))
    assert all(frac_of_bf16(T_bits[m, r]) == T_exact[m][r] for m in range(M) for r in range(R))
    Y = orc.linear_from_packed(res.values, res.meta, res.scale, T_bits, W, LA, K)
    Y_bf = brute_force_layer(Xb, W, LA, LB)
    # the LoRA part is a sizeable share of every row
    Yr = np.array([[float(sum(T_exact[m][r] * frac_of_bf16(LA[n, r]) for r in range(R)))
                    for n in range(N)] for m in range(M)])
    assert np.all(np.linalg.norm(Yr, axis=1) > 0.2 * np.linalg.norm(Y_bf, axis=1))
    np.testing.assert_allclose(Y, Y_bf, rtol=1e-12, atol=1e-12)


def test_meta_pack_unpack_round_trip():
    Xb = make_activation("heavy", 5, 128, seed=12)
    idx = orc.select_top2_of_4(Xb)
    np.testing.assert_array_equal(orc.unpack_meta(orc.pack_meta(idx), 128), idx)
    codes = orc.pack_meta(idx)
    lo = codes & 0xF
    assert set(np.unique(lo).tolist()) <= {4, 8, 12, 9, 13, 14}


# ---------------------------------------------------------------------------
# storage order of the packed operand (tiles of 16 rows x 64 channels)
# ---------------------------------------------------------------------------
def test_tiled_storage_offsets_by_hand():
    """Offsets written out from the format definition for M = 20, K = 192:
    Mp = 32, 3 steps; value j of row m at ((m//16)*3 + j//32)*512 + (m%16)*32 + j%32,
    meta byte j of row m at ((m//16)*3 + j//8)*128 + (m%16)*8 + j%8."""
    M, K = 20, 192
    vals = (np.arange(M * K // 2) % 65521).astype(np.uint16).reshape(M, K // 2)
    meta = (np.arange(M * K // 8) % 251).astype(np.uint8).reshape(M, K // 8)
    tv = orc.tile_rows(vals, K, 0).reshape(-1)
    tm = orc.tile_rows(meta, K, 0x44).reshape(-1)
    assert tv.size == 32 * K // 2 and tm.size == 32 * K // 8
    assert tv[(1 * 3 + 1) * 512 + 1 * 32 + 8] == vals[17, 40]     # m=17, j=40
    assert tv[(0 * 3 + 2) * 512 + 5 * 32 + 31] == vals[5, 95]     # m=5, j=95
    assert tm[(0 * 3 + 1) * 128 + 5 * 8 + 5] == meta[5, 13]       # m=5, j=13
    assert tm[(1 * 3 + 2) * 128 + 3 * 8 + 7] == meta[19, 23]      # m=19, j=23
    # padding rows 20..31 of the second block: zero values, meta 0x44
    assert tv[(1 * 3 + 0) * 512 + 4 * 32] == 0 and tm[(1 * 3 + 2) * 128 + 15 * 8] == 0x44
    np.testing.assert_array_equal(orc.untile_rows(orc.tile_rows(vals, K, 0), M, K), vals)


# ---- selective layer skipping (oracle reading 7) ----------------------------
def test_sequence_skipped_layer_is_the_textbook_product():
    """A skipped layer is X W^T, summed by hand over K; a sparse one equals
    linear_sparse_lora; the layers do not interact."""
    rng = np.random.default_rng(7)
    from workloads.generators import bf16_bits_from_f32
    X = bf16_bits_from_f32(rng.standard_normal((3, 8)).astype(np.float32))
    W = bf16_bits_from_f32(rng.standard_normal((5, 8)).astype(np.float32))
    LA = bf16_bits_from_f32(0.1 * rng.standard_normal((5, 2)).astype(np.float32))
    LB = bf16_bits_from_f32(0.1 * rng.standard_normal((2, 8)).astype(np.float32))
    x, w = orc.decode_bf16(X), orc.decode_bf16(W)
    by_hand = np.array([[sum(x[m, k] * w[n, k] for k in range(8)) for n in range(5)]
                        for m in range(3)])
    skipped, sparse = orc.linear_sequence([(X, W, LA, LB, True), (X, W, LA, LB, False)])
    assert np.array_equal(skipped, by_hand)
    assert np.array_equal(sparse, orc.linear_sparse_lora(X, W, LA, LB))
    # dense inputs that are exactly 2-sparse with no LoRA make both modes agree
    X2 = X.copy()
    X2[:, 2::4] = 0
    X2[:, 3::4] = 0
    a, b = orc.linear_sequence([(X2, W, None, None, True), (X2, W, None, None, False)])
    assert np.allclose(a, b, rtol=0, atol=1e-12)
