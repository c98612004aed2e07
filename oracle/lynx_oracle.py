"""Plain fp64 CPU oracle of the RT-Lynx sparse + LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the package entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code,
table or constant with the HIP library.

Source of the method: the RT-Lynx page (aitrends.kr, "RT-Lynx: Diffusion
Transformers에서 GEMM Sparsity를 Activation으로 옮겨 실현하는 방법").
  * 방법론, "핵심 메커니즘": Top-K based 2:4 selection of the activation gives
    X~; S(X) = s * X~; Ys = S(X) W^T, Yr = X (LA LB)^T, Y = Ys + Yr; the 2:4
    activation reaches the kernel in the sparse-tensor-core operand format.
  * 코드 예제, first formula: s = ||X||_2 / (||X~||_2 + eps).
  * 코드 예제, second formula: Y = Ys + Yr = S(X) W^T + X (LA LB)^T.
  * 핵심 아이디어 이해하기 / 용어 해설 "Norm Compensation": s restores the
    L2 norm of the dense activation; activations are per token, so the norm
    is taken per row (token).
  * 방법론, "구현 및 학습 세부": LoRA rank R = 64.

Readings where the page is silent or garbled (each also listed in the design
notes of the repository):
  1. Groups are 4 consecutive input channels (the reduction axis K), aligned
     at multiples of 4, as a 2:4 operand of a sparse matrix unit requires.
  2. Top-2 by |x|; equal magnitudes go to the lower channel index; -0 == +0.
     Every group keeps exactly two positions, even when it has fewer than two
     nonzeros.
  3. eps is taken as 0, with s = 1 for an all-zero row (the only case where
     ||X~|| = 0, since the top 2 of 4 keep at least half of each group's
     energy).  Then ||S(x)|| == ||x|| exactly in real arithmetic.
  4. The LoRA branch sees the dense, unscaled X, and is evaluated as
     (X LB^T) LA^T with LA [N x R], LB [R x K]; LA LB is never formed.
  5. No bias term.
  6. The packed format is the one the gfx950 sparse MFMA reads for its A
     operand (see pack_meta): kept values in ascending channel order, and a
     4-bit code per group, first kept position in bits 0-1, second in bits
     2-3, two groups per byte with the even group in the low nibble.  In
     memory both are stored in tiles of 16 rows x 64 channels (the operand
     tile of one v_smfmac_f32_16x16x64_bf16 step): see tile_rows.
  7. Selective Layer Skipping (방법론 "핵심 메커니즘"; 구현 및 학습 세부: in
     single-stream blocks layers such as Out/OUp are left out): a skipped
     layer is the original dense layer X W^T, without the LoRA branch, which
     only exists to correct the sparse one.  See linear_sequence.

Everything is computed in fp64 from exactly decoded bf16 inputs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# bf16 decoding (the inputs are bf16 bit patterns, uint16)
# ----------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> exact fp64 value.

    bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits
    (bias 127), 7 fraction bits.  Decoded directly from that definition.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    exp = (b >> 7) & 0xFF
    frac = (b & 0x7F).astype(np.float64)
    normal = sign * (1.0 + frac / 128.0) * np.exp2(exp.astype(np.float64) - 127.0)
    subnormal = sign * (frac / 128.0) * np.exp2(-126.0)
    out = np.where(exp == 0, subnormal, normal)
    if np.any(exp == 0xFF):
        raise ValueError("non-finite bf16 input is outside the layer's contract")
    return out


# ----------------------------------------------------------------------------
# Step 1: Top-K 2:4 selection (방법론, "핵심 메커니즘")
# ----------------------------------------------------------------------------
def select_top2_of_4(X_bits: np.ndarray) -> np.ndarray:
    """Indices of the two kept channels of every group of 4.

    Returns int64 [M, K/4, 2] with idx[..., 0] < idx[..., 1], positions 0..3
    inside the group.  Order: larger |x| first, equal |x| -> lower index
    (a stable sort on -|x|); then the pair is put in ascending order.
    """
    x = decode_bf16(X_bits)
    M, K = x.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    mag = np.abs(x).reshape(M, K // 4, 4)
    order = np.argsort(-mag, axis=-1, kind="stable")
    top2 = order[..., :2]
    return np.sort(top2, axis=-1).astype(np.int64)


def keep_mask(idx: np.ndarray) -> np.ndarray:
    """Boolean mask [M, K] of the kept channels, from select_top2_of_4."""
    M, G, _ = idx.shape
    mask = np.zeros((M, G, 4), dtype=bool)
    rows = np.arange(M)[:, None]
    groups = np.arange(G)[None, :]
    mask[rows, groups, idx[..., 0]] = True
    mask[rows, groups, idx[..., 1]] = True
    return mask.reshape(M, G * 4)


# ----------------------------------------------------------------------------
# Step 2: Norm Compensation (코드 예제, first formula)
# ----------------------------------------------------------------------------
def norm_scale(x: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """s[m] = ||x_m|| / ||x~_m|| in fp64, with s = 1 for a zero row (eps = 0)."""
    n2 = np.sum(x * x, axis=1)
    xt = np.where(mask, x, 0.0)
    nt2 = np.sum(xt * xt, axis=1)
    s = np.ones_like(n2)
    nz = nt2 > 0
    s[nz] = np.sqrt(n2[nz] / nt2[nz])
    return s


# ----------------------------------------------------------------------------
# Step 3: compressed operand (values + metadata)
# ----------------------------------------------------------------------------
def pack_values(X_bits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Kept bf16 bit patterns, unscaled, in ascending channel order: [M, K/2]."""
    Xb = np.asarray(X_bits, dtype=np.uint16)
    M, K = Xb.shape
    grp = Xb.reshape(M, K // 4, 4)
    kept = np.take_along_axis(grp, idx, axis=-1)  # [M, K/4, 2]
    return kept.reshape(M, K // 2).astype(np.uint16)


def pack_meta(idx: np.ndarray) -> np.ndarray:
    """4-bit code per group (i0 | i1 << 2), two groups per byte: [M, K/8] uint8.

    Group 2j sits in the low nibble of byte j, group 2j+1 in the high nibble.
    Read as little-endian 16-bit words, the code of group g of a 16-channel
    block sits at bits 4g..4g+3: this is the sparse-index word of one lane of
    the gfx950 SMFMAC A operand.
    """
    M, G, _ = idx.shape
    if G % 2:
        raise ValueError("K must be a multiple of 8 to pack metadata")
    code = (idx[..., 0] | (idx[..., 1] << 2)).astype(np.uint8)  # [M, G]
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)


def unpack_meta(meta: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_meta: [M, K/8] uint8 -> int64 [M, K/4, 2]."""
    m = np.asarray(meta, dtype=np.uint8).astype(np.int64)
    M = m.shape[0]
    code = np.empty((M, K // 4), dtype=np.int64)
    code[:, 0::2] = m & 0xF
    code[:, 1::2] = m >> 4
    return np.stack([code & 3, code >> 2], axis=-1)


def unpack_dense(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Rebuild X~ (fp64, zeros at dropped channels) from the packed operand."""
    idx = unpack_meta(meta, K)
    v = decode_bf16(values).reshape(values.shape[0], K // 4, 2)
    out = np.zeros((values.shape[0], K // 4, 4))
    rows = np.arange(values.shape[0])[:, None]
    groups = np.arange(K // 4)[None, :]
    # assignment order matters only if i0 == i1, which the format forbids
    out[rows, groups, idx[..., 0]] = v[..., 0]
    out[rows, groups, idx[..., 1]] = v[..., 1]
    return out.reshape(values.shape[0], K)


# ----------------------------------------------------------------------------
# Storage order of the packed operand: 16-row x 64-channel tiles
# ----------------------------------------------------------------------------
TILE_ROWS = 16
TILE_CHANNELS = 64


def padded_rows(M: int) -> int:
    """Rows of the stored packed operand: M rounded up to a multiple of 16."""
    return -(-M // TILE_ROWS) * TILE_ROWS


def tile_rows(rowmajor: np.ndarray, K: int, pad_value: int) -> np.ndarray:
    """Row-major per-row data [M, K * w / 64] -> stored order.

    The stored order is [ceil(M/16)][K/64][16][w]: for each block of 16 rows
    and each 64-channel step, the 16 rows' w items of that step (w = 32 kept
    values, or 8 metadata bytes) are contiguous, row after row.  Rows past M
    in the last block hold pad_value.
    """
    M, L = rowmajor.shape
    w = L * TILE_CHANNELS // K
    Mp = padded_rows(M)
    full = np.full((Mp, L), pad_value, dtype=rowmajor.dtype)
    full[:M] = rowmajor
    return full.reshape(Mp // 16, 16, K // 64, w).transpose(0, 2, 1, 3).copy()


def untile_rows(stored: np.ndarray, M: int, K: int) -> np.ndarray:
    """Inverse of tile_rows (padding dropped): -> row-major [M, K * w / 64]."""
    nb, steps, rows, w = stored.shape
    return stored.transpose(0, 2, 1, 3).reshape(nb * rows, steps * w)[:M]


# ----------------------------------------------------------------------------
# The whole sparsifier and the layer (방법론, "핵심 메커니즘"; 코드 예제)
# ----------------------------------------------------------------------------
@dataclass
class SparsifyResult:
    idx: np.ndarray      # int64 [M, K/4, 2]
    values: np.ndarray   # uint16 [M, K/2] (bf16 bits, unscaled), row-major
    meta: np.ndarray     # uint8 [M, K/8], row-major
    scale: np.ndarray    # fp64 [M]
    T: np.ndarray | None  # fp64 [M, R] = X LB^T, or None without LoRA

    def values_stored(self) -> np.ndarray:
        """values in stored order, padding rows zero (flat, uint16)."""
        K = self.values.shape[1] * 2
        return tile_rows(self.values, K, 0).reshape(-1)

    def meta_stored(self) -> np.ndarray:
        """meta in stored order, padding rows coded (0,1),(0,1) = 0x44 (flat)."""
        K = self.meta.shape[1] * 8
        return tile_rows(self.meta, K, 0x44).reshape(-1)


def sparsify(X_bits: np.ndarray, LB_bits: np.ndarray | None = None) -> SparsifyResult:
    """Selection, norm scale, packing and the LoRA down-projection T = X LB^T."""
    x = decode_bf16(X_bits)
    idx = select_top2_of_4(X_bits)
    mask = keep_mask(idx)
    s = norm_scale(x, mask)
    T = None if LB_bits is None else x @ decode_bf16(LB_bits).T
    return SparsifyResult(idx, pack_values(X_bits, idx), pack_meta(idx), s, T)


def linear_sparse_lora(X_bits, W_bits, LA_bits=None, LB_bits=None) -> np.ndarray:
    """Y = s * (X~ W^T) + (X LB^T) LA^T, fp64 [M, N].

    s * (X~ W^T) equals (s X~) W^T = S(X) W^T; the LoRA term uses dense X.
    Rows of X may be any subset of a larger X: the layer is row-independent.
    """
    x = decode_bf16(X_bits)
    mask = keep_mask(select_top2_of_4(X_bits))
    s = norm_scale(x, mask)
    xt = np.where(mask, x, 0.0)
    Y = s[:, None] * (xt @ decode_bf16(W_bits).T)
    if LA_bits is not None and LB_bits is not None:
        T = x @ decode_bf16(LB_bits).T
        Y = Y + T @ decode_bf16(LA_bits).T
    return Y


def linear_from_packed(values, meta, scale, T_bits, W_bits, LA_bits, K: int) -> np.ndarray:
    """Y from an already packed operand: scale * (X~ W^T) + T LA^T, fp64.

    This is the layer with the sparsifier's outputs given as inputs (scale as
    given, T as bf16 bits or None).
    """
    xt = unpack_dense(values, meta, K)
    Y = np.asarray(scale, dtype=np.float64)[:, None] * (xt @ decode_bf16(W_bits).T)
    if T_bits is not None and LA_bits is not None:
        Y = Y + decode_bf16(T_bits) @ decode_bf16(LA_bits).T
    return Y


def linear_dense(X_bits, W_bits) -> np.ndarray:
    """The dense layer X W^T the speedup is measured against, fp64 [M, N]."""
    return decode_bf16(X_bits) @ decode_bf16(W_bits).T


def linear_sequence(layers) -> list:
    """Outputs of a sequence of layers, each sparse + LoRA or skipped (dense).

    layers: iterable of (X_bits, W_bits, LA_bits, LB_bits, skipped).  A
    skipped layer is X W^T (reading 7); the others are linear_sparse_lora.
    The layers are independent: the sequence is the block's linears in order,
    without the attention and activation functions between them.
    """
    out = []
    for X_bits, W_bits, LA_bits, LB_bits, skipped in layers:
        if skipped:
            out.append(linear_dense(X_bits, W_bits))
        else:
            out.append(linear_sparse_lora(X_bits, W_bits, LA_bits, LB_bits))
    return out

