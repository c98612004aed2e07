"""Synthetic fidelity study of the RT-Lynx layer (CPU, fp64; the GPU check is
in test_fidelity.py).

What the page claims and what is measured here, on the synthetic activation
distributions of the workloads (heavy-tailed channels; post-GELU), with
W ~ N(0, 1/K):
  * 핵심 아이디어 이해하기 (출발점): weights are quasi-Gaussian while each
    token's activation is carried by few channels, so 2:4 sparsity on the
    activation gives a smaller output error than 2:4 sparsity on the weight.
  * 해결 원리 / 핵심 기여: S(X) = s X~ restores the dense activation's L2
    norm (Norm Compensation), and a rank-R LoRA branch fitted to the residual
    recovers what sparsification lost.
  * 구현 및 학습 세부: LA, LB minimise ||X W^T - (S(X) W^T + X (LA LB)^T)||^2,
    R = 64.  The page trains them by distillation; here the same loss is
    minimised in closed form on calibration activations (reduced-rank
    regression), and the result is scored on held-out activations.

Variants, each scored by the relative Frobenius error of Y against the dense
layer and by the ratio of row norms (how well the output's scale survives):
  SA        2:4 activation, s = 1                      (no compensation)
  SA+NC     2:4 activation, s = ||x|| / ||x~||         (the method without LoRA)
  SA+NC+L   the method                                 (S(X) W^T + X (LA LB)^T)
  SA+L      2:4 activation with LoRA, s = 1
  SW        2:4 weight (top-2 |w| of 4 along K per output)
  SW+L      2:4 weight with a LoRA fitted the same way

    python -m tests.fidelity_study          # prints the table (under a minute)
"""
from __future__ import annotations

import numpy as np

from oracle import lynx_oracle as orc
from workloads import bf16_bits_from_f32, make_activation, make_weights


def fit_lora(X: np.ndarray, E: np.ndarray, R: int, ridge: float = 1e-8):
    """Rank-R Q = LB^T LA^T minimising ||E - X Q||_F (reduced-rank regression).

    Q_ols = (X^T X)^-1 X^T E; the best rank-R fit projects the fitted values
    X Q_ols onto their top R right singular vectors V_R: Q = Q_ols V_R V_R^T.
    Returns LA [N, R] = V_R and LB [R, K] = (Q_ols V_R)^T.
    """
    G = X.T @ X
    G[np.diag_indices_from(G)] += ridge * np.trace(G) / G.shape[0]
    Q_ols = np.linalg.solve(G, X.T @ E)
    _, _, Vt = np.linalg.svd(X @ Q_ols, full_matrices=False)
    V = Vt[:R].T
    return V, (Q_ols @ V).T


def weight_2of4(W_bits: np.ndarray) -> np.ndarray:
    """2:4 weight: per output row, the top 2 |w| of every 4 consecutive K."""
    keep = orc.keep_mask(orc.select_top2_of_4(W_bits))
    return np.where(keep, orc.decode_bf16(W_bits), 0.0)


def sparse_parts(X_bits: np.ndarray):
    """(x, x~, s) of the oracle: dense activation, kept channels, norm scale."""
    x = orc.decode_bf16(X_bits)
    mask = orc.keep_mask(orc.select_top2_of_4(X_bits))
    return x, np.where(mask, x, 0.0), orc.norm_scale(x, mask)


def score(Y: np.ndarray, Yd: np.ndarray) -> dict:
    rel = float(np.linalg.norm(Y - Yd) / np.linalg.norm(Yd))
    ratio = np.linalg.norm(Y, axis=1) / np.linalg.norm(Yd, axis=1)
    return {"rel_err": rel, "norm_ratio": float(np.mean(ratio))}


def study(kind: str, K: int = 1024, N: int = 512, M_cal: int = 16384, M_eval: int = 2048,
          R: int = 64, seed: int = 0, ridge: float = 1e-4) -> dict:
    """All variants for one activation distribution; returns name -> score,
    plus the fitted method's LoRA factors and the evaluation inputs.

    Calibration and evaluation rows are tokens of the same layer: one draw of
    the channel scales and outlier channels, split into M_cal + M_eval rows
    (the fit would not transfer between layers with different scales).
    Calibration needs M_cal >> K for the regression to generalise."""
    X_bits = make_activation(kind, M_cal + M_eval, K, seed)
    Xc_bits, Xe_bits = X_bits[:M_cal], X_bits[M_cal:]
    W_bits, _, _ = make_weights(N, K, R, seed)
    w = orc.decode_bf16(W_bits)
    ws = weight_2of4(W_bits)

    xc, xtc, sc = sparse_parts(Xc_bits)
    xe, xte, se = sparse_parts(Xe_bits)
    Yd_c, Yd_e = xc @ w.T, xe @ w.T

    out = {}
    out["SA"] = score(xte @ w.T, Yd_e)
    out["SA+NC"] = score(se[:, None] * (xte @ w.T), Yd_e)
    # LoRA on the method's residual (with NC), fitted on calibration rows
    LA, LB = fit_lora(xc, Yd_c - sc[:, None] * (xtc @ w.T), R, ridge)
    out["SA+NC+L"] = score(se[:, None] * (xte @ w.T) + (xe @ LB.T) @ LA.T, Yd_e)
    LA0, LB0 = fit_lora(xc, Yd_c - xtc @ w.T, R, ridge)
    out["SA+L"] = score(xte @ w.T + (xe @ LB0.T) @ LA0.T, Yd_e)
    out["SW"] = score(xe @ ws.T, Yd_e)
    LAw, LBw = fit_lora(xc, Yd_c - xc @ ws.T, R, ridge)
    out["SW+L"] = score(xe @ ws.T + (xe @ LBw.T) @ LAw.T, Yd_e)
    out["_lora"] = (LA, LB)
    out["_eval"] = (Xe_bits, W_bits)
    return out


def lora_bits(LA: np.ndarray, LB: np.ndarray):
    """The fitted factors as bf16 bits, with the scale moved so both factors
    are O(1) before rounding (LA LB is unchanged)."""
    a = np.sqrt(np.abs(LB).max() / max(np.abs(LA).max(), 1e-30))
    return (bf16_bits_from_f32((LA * a).astype(np.float32)),
            bf16_bits_from_f32((LB / a).astype(np.float32)))


def main():
    names = ["SA", "SA+NC", "SA+NC+L", "SA+L", "SW", "SW+L"]
    print("| activations | " + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    for kind in ("heavy", "gelu"):
        res = study(kind)
        cells = [f"{res[n]['rel_err']:.4f} ({res[n]['norm_ratio']:.3f})" for n in names]
        print(f"| {kind} | " + " | ".join(cells) + " |")


if __name__ == "__main__":
    main()
