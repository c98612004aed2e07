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
