"""Plain fp64 CPU oracle of block-sparse attention with block routing and a
dropped-block residual.  TEST INFRASTRUCTURE ONLY: nothing on the product path
imports this; only tests, the smoke check and the benchmark's CPU-baseline leg
do.  It shares no code with the HIP library or its Python binding.

What it computes (per batch entry b and head h, tokens [N, d]):

  pool     Mean of the queries of each query block and of the keys and values of
           each key block, over the block's actual tokens (the last block may be
           short).  Centroid estimation of block importance, PARK page,
           section 4.1 (query- and key-centroid estimates).
  proxy    s_IJ = scale * qbar_I . kbar_J and P_I. = softmax over J of s_I.
           ("block proxy scores", Sol-Attn abstract; block importance
           normalised across key blocks, PARK page, section 3.2).
  select   Compare a per-block quantity r_IJ with tau (Sol-Attn abstract:
           blocks are chosen by comparing proxy scores against a threshold
           during online softmax).  Two readings:
             RELATIVE  r = P_IJ / max_J' P_IJ' = exp(s_IJ - max_J' s_IJ')
             ABSOLUTE  r = P_IJ
             TOPP      r = P_IJ, and C_I is the shortest prefix of the ranking
                       (r descending, J ascending) whose proxy mass reaches
                       1 - tau: J is a candidate iff the mass ranked before it
                       is < 1 - tau (cumulative-mass retention, the dynamic
                       budget the Sol-Attn abstract contrasts with fixed ones)
           candidates C_I = {J : r_IJ >= tau} (RELATIVE, ABSOLUTE); a top-k
           budget caps |C_I| at
           max_keep (rank by r descending, then J ascending); if fewer than
           min_keep clear tau, the first min_keep of the ranking are kept; key
           blocks that start inside the dense prefix are always kept, and a
           query block that starts inside the prefix keeps every key block.
  forward  For each query row i of block I, exact logits a_it = scale q_i.k_t over
           the tokens t of kept blocks, and one residual logit per dropped block
           b_iJ = scale q_i.kbar_J + ln n_J standing for its n_J tokens with the
           block-mean key and value ("reusing the proxy scores of unselected
           blocks to approximate their contribution", Sol-Attn abstract).  Both
           share one max and one normaliser:
             o_i = (sum_t e^{a_it - M} v_t + sum_J e^{b_iJ - M} vbar_J) / Z,
             LSE_i = M + ln Z.
           When every key of block J equals kbar_J the residual term is exact;
           otherwise it is a lower bound on the block's log-mass (Jensen; PARK
           page, appendix D.2).

Everything is float64 numpy; inputs of any float dtype are upcast exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

RELATIVE = 0
ABSOLUTE = 1
TOPP = 2
CENTROID = 0            # proxy: softmax over key blocks of the query block mean's scores
PAMA = 1                # proxy: per-query softmax over key blocks, averaged in the query block
EXEMPT_BAND = 1e-4      # |r - cut| below this: the keep decision is rounding-sensitive


@dataclass
class RouteParams:
    block_q: int
    block_k: int
    tau: float
    tau_mode: int = RELATIVE
    max_keep: int = 0          # 0 = no cap
    min_keep: int = 1
    n_prefix: int = 0          # dense-attended leading tokens
    scale: float = 0.0         # 0 => 1/sqrt(d)
    proxy: int = CENTROID      # CENTROID or PAMA

    def sigma(self, d: int) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(d)


def n_blocks(N: int, bs: int) -> int:
    return -(-N // bs)


def block_counts(N: int, bs: int) -> np.ndarray:
    starts = np.arange(n_blocks(N, bs)) * bs
    return np.minimum(starts + bs, N) - starts


def pool(X: np.ndarray, bs: int) -> np.ndarray:
    """Block means over the actual tokens of each block: [ceil(N/bs), d]."""
    X = np.asarray(X, dtype=np.float64)
    N, d = X.shape
    nb = n_blocks(N, bs)
    out = np.empty((nb, d))
    for J in range(nb):
        out[J] = X[J * bs:min((J + 1) * bs, N)].mean(axis=0)
    return out


def proxy_scores(qbar: np.ndarray, kbar: np.ndarray, sigma: float) -> np.ndarray:
    """s[I, J] = sigma * qbar_I . kbar_J."""
    return sigma * (qbar @ kbar.T)


def pama_importance(q: np.ndarray, kbar: np.ndarray, bq: int, sigma: float) -> np.ndarray:
    """A[I, J] = mean over the queries i of query block I of softmax_J(sigma q_i . kbar_J).

    Per-query attention-mass aggregation (PARK page, section 5.1): every
    original query normalises its attention over the key-block centroids on its
    own, and the distributions are averaged within the query block (instead of
    averaging the queries first).  Rows sum to 1.  Reading: the softmax runs over
    the centroids with equal weight, like the centroid proxy (no block-size
    weight for a short last key block)."""
    q = np.asarray(q, dtype=np.float64)
    logits = sigma * (q @ kbar.T)                        # [N, n_kb]
    logits -= logits.max(axis=1, keepdims=True)
    P = np.exp(logits)
    P /= P.sum(axis=1, keepdims=True)
    N = q.shape[0]
    return np.stack([P[I * bq:min((I + 1) * bq, N)].mean(axis=0) for I in range(n_blocks(N, bq))])


def _logsumexp_rows(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]


def compare_quantity(s: np.ndarray, tau_mode: int) -> np.ndarray:
    """r[I, J]: P/max P (RELATIVE), else the proxy probability P."""
    if tau_mode == RELATIVE:
        return np.exp(s - s.max(axis=1, keepdims=True))
    if tau_mode in (ABSOLUTE, TOPP):
        return np.exp(s - _logsumexp_rows(s)[:, None])
    raise ValueError(f"unknown tau_mode {tau_mode}")


def rank_order(r_row: np.ndarray) -> np.ndarray:
    """Key blocks ordered by r descending, ties by J ascending."""
    J = np.arange(r_row.shape[0])
    return np.lexsort((J, -r_row))


@dataclass
class RouteResult:
    mask: np.ndarray            # bool [n_qb, n_kb]
    s: np.ndarray               # proxy scores [n_qb, n_kb]
    r: np.ndarray               # compared quantity [n_qb, n_kb]
    row_max: np.ndarray         # max_J s [n_qb]
    row_lse: np.ndarray         # logsumexp_J s [n_qb]
    exempt: np.ndarray          # bool [n_qb, n_kb]: decision within EXEMPT_BAND of its cut
    qbar: np.ndarray = field(repr=False, default=None)
    kbar: np.ndarray = field(repr=False, default=None)
    vbar: np.ndarray = field(repr=False, default=None)

    @property
    def kv_count(self) -> np.ndarray:
        return self.mask.sum(axis=1).astype(np.int64)

    def kv_list(self, I: int) -> np.ndarray:
        return np.flatnonzero(self.mask[I])


def select(r: np.ndarray, p: RouteParams, N: int) -> tuple:
    """Keep mask and rounding-exemption mask from r (see module docstring)."""
    n_qb, n_kb = r.shape
    mask = np.zeros((n_qb, n_kb), dtype=bool)
    exempt = np.zeros((n_qb, n_kb), dtype=bool)
    prefix_kb = np.arange(n_kb) * p.block_k < p.n_prefix
    for I in range(n_qb):
        row = r[I]
        order = rank_order(row)
        if p.tau_mode == TOPP:
            # keep rank i iff the mass ranked before it is below 1 - tau
            target = 1.0 - p.tau
            before = np.concatenate([[0.0], np.cumsum(row[order])[:-1]])
            cand = np.zeros(n_kb, dtype=bool)
            cand[order[before < target]] = True
            exempt[I, order[np.abs(before - target) < EXEMPT_BAND]] = True
        else:
            cand = row >= p.tau
            exempt[I] |= np.abs(row - p.tau) < EXEMPT_BAND
        n_c = int(cand.sum())
        if p.max_keep > 0 and n_c > p.max_keep:
            # candidates are a prefix of the ranking; keep its first max_keep
            keep = order[:p.max_keep]
            cut = row[order[p.max_keep - 1]]
            exempt[I] |= np.abs(row - cut) < EXEMPT_BAND
        elif n_c < p.min_keep:
            keep = order[:min(p.min_keep, n_kb)]
            cut = row[order[min(p.min_keep, n_kb) - 1]]
            exempt[I] |= np.abs(row - cut) < EXEMPT_BAND
        else:
            keep = np.flatnonzero(cand)
        mask[I, keep] = True
        mask[I] |= prefix_kb
        if I * p.block_q < p.n_prefix:
            mask[I] = True
        exempt[I] &= ~(prefix_kb | (I * p.block_q < p.n_prefix))
    return mask, exempt


def route_ref(q: np.ndarray, k: np.ndarray, p: RouteParams) -> RouteResult:
    """Routing for one head.  q, k: [N, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, d = q.shape
    qbar = pool(q, p.block_q)
    kbar = pool(k, p.block_k)
    if p.proxy == PAMA:
        # scores whose softmax is the importance A (rows of A sum to 1): s = ln A
        with np.errstate(divide="ignore"):
            s = np.log(pama_importance(q, kbar, p.block_q, p.sigma(d)))
    else:
        s = proxy_scores(qbar, kbar, p.sigma(d))
    r = compare_quantity(s, p.tau_mode)
    mask, exempt = select(r, p, N)
    return RouteResult(mask=mask, s=s, r=r, row_max=s.max(axis=1), row_lse=_logsumexp_rows(s),
                       exempt=exempt, qbar=qbar, kbar=kbar)


def _kept_tokens(mask_row: np.ndarray, bk: int, N: int) -> np.ndarray:
    blocks = np.flatnonzero(mask_row)
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(J * bk, min((J + 1) * bk, N)) for J in blocks])


def forward_ref_with_mask(q, k, v, mask: np.ndarray, p: RouteParams, rows=None,
                          return_weights: bool = False, residual: bool = True):
    """Sparse attention with residual for one head, under a given keep mask [n_qb, n_kb].

    rows: optional iterable of query-block indices to evaluate (others left NaN).
    residual=False drops the dropped blocks entirely (attention over kept tokens only).
    Returns (O [N, d], LSE [N]) and, with return_weights, a list per query block of
    (token_idx, w_tokens [m_I, n_t], dropped_blocks, w_blocks [m_I, n_d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    sig = p.sigma(d)
    kbar = pool(k, p.block_k)
    vbar = pool(v, p.block_k)
    n_j = block_counts(N, p.block_k).astype(np.float64)
    O = np.full((N, d), np.nan)
    L = np.full(N, np.nan)
    weights = []
    blocks = range(n_blocks(N, p.block_q)) if rows is None else rows
    for I in blocks:
        i0, i1 = I * p.block_q, min((I + 1) * p.block_q, N)
        qi = q[i0:i1]
        tok = _kept_tokens(mask[I], p.block_k, N)
        dropped = np.flatnonzero(~mask[I]) if residual else np.zeros(0, dtype=np.int64)
        a = sig * (qi @ k[tok].T)                                    # exact logits
        b = sig * (qi @ kbar[dropped].T) + np.log(n_j[dropped])[None, :]   # residual logits
        M = np.full(i1 - i0, -np.inf)
        if a.size:
            M = np.maximum(M, a.max(axis=1))
        if b.size:
            M = np.maximum(M, b.max(axis=1))
        ea = np.exp(a - M[:, None])
        eb = np.exp(b - M[:, None])
        Z = ea.sum(axis=1) + eb.sum(axis=1)
        O[i0:i1] = (ea @ v[tok] + eb @ vbar[dropped]) / Z[:, None]
        L[i0:i1] = M + np.log(Z)
        if return_weights:
            weights.append((tok, ea / Z[:, None], dropped, eb / Z[:, None]))
    if return_weights:
        return O, L, weights
    return O, L


def forward_ref(q, k, v, p: RouteParams, rows=None, return_route: bool = False):
    """Routing followed by sparse attention with residual, one head."""
    rt = route_ref(q, k, p)
    O, L = forward_ref_with_mask(q, k, v, rt.mask, p, rows=rows)
    if return_route:
        return O, L, rt
    return O, L


def dense_ref(q, k, v, scale: float = 0.0, rows=None, chunk: int = 1024):
    """Plain softmax attention for one head (no routing): O [N, d], LSE [N].
    rows: optional (start, stop) token range."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    sig = scale if scale > 0 else 1.0 / math.sqrt(d)
    r0, r1 = (0, N) if rows is None else rows
    O = np.empty((r1 - r0, d))
    L = np.empty(r1 - r0)
    for c0 in range(r0, r1, chunk):
        c1 = min(c0 + chunk, r1)
        S = sig * (q[c0:c1] @ k.T)
        M = S.max(axis=1, keepdims=True)
        E = np.exp(S - M)
        Z = E.sum(axis=1, keepdims=True)
        O[c0 - r0:c1 - r0] = (E @ v) / Z
        L[c0 - r0:c1 - r0] = (M + np.log(Z))[:, 0]
    return O, L


def attention_recall(q, k, mask: np.ndarray, p: RouteParams) -> float:
    """Share of dense softmax weight that falls in kept blocks (PARK page, section 3.2).
    A diagnostic for small inputs only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, d = q.shape
    S = p.sigma(d) * (q @ k.T)
    W = np.exp(S - S.max(axis=1, keepdims=True))
    W /= W.sum(axis=1, keepdims=True)
    qb = np.arange(N) // p.block_q
    kb = np.arange(N) // p.block_k
    keep = mask[qb][:, kb]
    return float((W * keep).sum() / N)
