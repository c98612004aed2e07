"""Helpers for the GPU tests: host<->device transfer of bf16 bit arrays and the
parity measures.  No arithmetic of the method lives here."""
import os
import sys

import numpy as np
import torch

ROW_REL_TOL = 5e-3     # per-row relative Frobenius error bound on Y and T
SCALE_REL_TOL = 1e-5   # |s_gpu / s_ref - 1|


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> contiguous bf16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


# Rows whose reference norm is below the bf16 normal range come only from
# subnormal inputs, which the matrix units may flush; they are compared against
# this floor instead of their own norm.  Exactly-zero reference rows must be 0.
NORM_FLOOR = 2.0 ** -96


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||got_m - ref_m|| / max(||ref_m||, floor) per row; rows with ref == 0
    report max|got| (so they pass only when exactly zero)."""
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    out = np.where(den > 0, num / np.maximum(den, NORM_FLOOR), np.abs(got).max(axis=1))
    return out


def report(name: str, got: np.ndarray, ref: np.ndarray) -> dict:
    """Parity summary: worst row error, cosine, max-abs, non-finite count."""
    err = row_rel_err(got, ref)
    cos = float(np.sum(got * ref) / max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300))
    rep = dict(name=name, max_row_rel=float(err.max()), mean_row_rel=float(err.mean()),
               cosine=cos, max_abs=float(np.abs(got - ref).max()),
               nonfinite=int((~np.isfinite(got)).sum()))
    say(f"{name}: {rep}")
    return rep


def sample_rows(M: int, n: int = 48, seed: int = 0, tile: int = 256) -> np.ndarray:
    """Rows spanning first/last tiles, tile boundaries and random interior rows."""
    rng = np.random.default_rng(seed)
    picks = {0, 1, M - 1, M - 2}
    for b in range(tile, M, tile * max(1, (M // tile) // 8)):
        picks |= {b - 1, b}
    picks |= set(rng.integers(0, M, size=n).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < M))


def dump_dir():
    """Directory for raw probe outputs kept for offline inspection, named by the
    LYNX_PROBE_DUMP_DIR environment variable; None (nothing is written) when
    it is unset."""
    d = os.environ.get("LYNX_PROBE_DUMP_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
    return d


# ---- calls with poisoned outputs -------------------------------------------
# Every output buffer (and the layer's workspace) is filled with a value no
# kernel writes from finite inputs before each call: a bf16 NaN, a fp32 NaN,
# meta bytes 0xFF (code 3|3<<2, which the format never uses).  An element the
# kernels fail to write then fails the parity checks instead of passing on
# whatever an earlier call left in a recycled buffer.
NAN_BF16_BITS = 0x7FC0


def nan_bf16(shape) -> torch.Tensor:
    return torch.full(shape, NAN_BF16_BITS, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def poisoned_bytes(n: int) -> torch.Tensor:
    return torch.full((max(n, 1),), 0xFF, dtype=torch.uint8, device="cuda")


def sparse_lora(X, W, LA=None, LB=None):
    import activation_sparse_gemm_amd as lynx
    (M, K), N = X.shape, W.shape[0]
    R = 0 if LA is None else LA.shape[1]
    return lynx.linear_sparse_lora(X, W, LA, LB, Y=nan_bf16((M, N)),
                                   workspace=poisoned_bytes(lynx.workspace_bytes(M, K, R)))


def sparse_lora_noalloc(X, W, LA=None, LB=None):
    import activation_sparse_gemm_amd as lynx
    return lynx.linear_sparse_lora_noalloc(X, W, LA, LB, Y=nan_bf16((X.shape[0], W.shape[0])))


def dense(X, W):
    import activation_sparse_gemm_amd as lynx
    return lynx.linear_dense(X, W, Y=nan_bf16((X.shape[0], W.shape[0])))


def packed(values, meta, scale, T, W, LA=None):
    import activation_sparse_gemm_amd as lynx
    return lynx.linear_sparse_lora_packed(values, meta, scale, T, W, LA,
                                          Y=nan_bf16((scale.shape[0], W.shape[0])))


def sparsify(X, LB=None):
    import activation_sparse_gemm_amd as lynx
    M, K = X.shape
    Mp = lynx.padded_rows(M) if hasattr(lynx, "padded_rows") else (M + 15) // 16 * 16
    out = dict(values=nan_bf16((Mp * K // 2,)),
               meta=torch.full((Mp * K // 8,), 0xFF, dtype=torch.uint8, device="cuda"),
               scale=torch.full((M,), float("nan"), dtype=torch.float32, device="cuda"))
    if LB is not None:
        out["T"] = nan_bf16((M, LB.shape[0]))
    return lynx.sparsify(X, LB, out=out)


def sequence(layers):
    """lynx_linear_sequence with every layer's Y and the workspace poisoned."""
    import activation_sparse_gemm_amd as lynx
    for d in layers:
        d["Y"].view(torch.int16).fill_(NAN_BF16_BITS)
    ws = poisoned_bytes(lynx.sequence_workspace_bytes(layers))
    lynx.linear_sequence(layers, workspace=ws)
