"""Oracle of the probe-fitted residual correction (SparsePR summary, section B:
probe selection, affine calibration, subspace restriction, correction).
TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline);
independent of the HIP library.  float64 numpy throughout.

For one head, under a keep mask:

  O_s    sparse attention over the kept tokens only (no block residual: the
         correction replaces the block-level approximation).
  probes P rows per query block, evenly spread: row I*bq + floor((j + 1/2) m_I / P),
         j < P, m_I the block's actual rows (stratified across query groups).
  O_d    exact dense attention at the probe rows.
  fit    X = O_s[probes], R = O_d[probes] - X.  The affine map R ~ b + x B is a
         ridge regression with an unpenalised intercept: with the column means
         xm, rm and the centred Xc, Rc,
             B = (Xc^T Xc + lam I)^-1 Xc^T Rc,   b = rm - xm B,
         lam = ridge * trace(Xc^T Xc) / d (a ridge relative to the data's scale).
  subspace  V_k: the k leading right singular vectors of R; Pk = V_k V_k^T.
  output rows that are probes take O_d; every other row takes
             O_s + (b + O_s B) Pk.

Readings (the summary gives no formulas): the probe spacing, the relative ridge,
the uncentred R for the subspace, and exact values at the probe rows.
"""
from __future__ import annotations

import numpy as np

from .sparse_attn_ref import RouteParams, dense_ref, forward_ref_with_mask, n_blocks


def probe_rows(N: int, bq: int, per_block: int) -> np.ndarray:
    rows = []
    for I in range(n_blocks(N, bq)):
        m = min(bq, N - I * bq)
        for j in range(per_block):
            rows.append(I * bq + int(np.floor((j + 0.5) * m / per_block)))
    return np.asarray(rows, dtype=np.int64)


def fit(X: np.ndarray, R: np.ndarray, ridge: float, rank: int):
    """(b [d], B [d, d], Pk [d, d]) from probe sparse outputs X and residuals R [M, d]."""
    X = np.asarray(X, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    d = X.shape[1]
    xm, rm = X.mean(axis=0), R.mean(axis=0)
    Xc, Rc = X - xm, R - rm
    G = Xc.T @ Xc
    lam = ridge * np.trace(G) / d
    B = np.linalg.solve(G + lam * np.eye(d), Xc.T @ Rc)
    b = rm - xm @ B
    _, _, Vt = np.linalg.svd(R, full_matrices=False)
    Vk = Vt[:rank].T
    return b, B, Vk @ Vk.T


def correct(Os: np.ndarray, Od_probe: np.ndarray, probes: np.ndarray, b, B, Pk) -> np.ndarray:
    out = Os + (b[None, :] + Os @ B) @ Pk
    out[probes] = Od_probe
    return out


def sparsepr_ref(q, k, v, mask: np.ndarray, p: RouteParams, per_block: int, rank: int, ridge: float):
    """Corrected output [N, d] of one head, plus the pieces (O_s, probes, O_d at probes, b, B, Pk)."""
    N, d = np.asarray(q).shape
    Os, _ = forward_ref_with_mask(q, k, v, mask, p, residual=False)
    probes = probe_rows(N, p.block_q, per_block)
    Od, _ = dense_ref(np.asarray(q, dtype=np.float64)[probes], k, v, scale=p.sigma(d))
    b, B, Pk = fit(Os[probes], Od - Os[probes], ridge, rank)
    return correct(Os, Od, probes, b, B, Pk), (Os, probes, Od, b, B, Pk)
