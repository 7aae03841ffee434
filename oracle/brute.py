"""Scalar brute-force oracle for tiny inputs.  TEST INFRASTRUCTURE ONLY.

A second, independent implementation of the same definitions as
sparse_attn_ref (routing by block means, threshold and budget, exact kept
tokens plus one residual logit per dropped block), written with explicit
Python loops over tokens, blocks and feature dimensions and exactly rounded
sums (math.fsum).  It exists to pin the vectorised oracle: the two must agree
to ~1e-12 on every tiny case.  Lists of lists in, lists out.
"""
from __future__ import annotations

import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def _block_ranges(N, bs):
    out = []
    start = 0
    while start < N:
        out.append((start, min(start + bs, N)))
        start += bs
    return out


def _mean_rows(X, lo, hi):
    d = len(X[0])
    n = hi - lo
    return [math.fsum(X[t][c] for t in range(lo, hi)) / n for c in range(d)]


def brute_pama(q, kbar, qlo, qhi, scale):
    """Importance of every key block for the query block [qlo, qhi): each query's
    softmax over the key-block means, averaged over the block's queries."""
    nk = len(kbar)
    acc = [[] for _ in range(nk)]
    for i in range(qlo, qhi):
        lg = [scale * _dot(q[i], kbar[J]) for J in range(nk)]
        top = max(lg)
        e = [math.exp(x - top) for x in lg]
        z = math.fsum(e)
        for J in range(nk):
            acc[J].append(e[J] / z)
    return [math.fsum(a) / (qhi - qlo) for a in acc]


def brute_route(q, k, block_q, block_k, tau, tau_mode, max_keep, min_keep, n_prefix, scale, pama=False):
    """Keep mask as a list of lists of bools [n_qb][n_kb].  pama: the proxy is the
    per-query block attention averaged in the query block."""
    N = len(q)
    qr = _block_ranges(N, block_q)
    kr = _block_ranges(N, block_k)
    qbar = [_mean_rows(q, lo, hi) for lo, hi in qr]
    kbar = [_mean_rows(k, lo, hi) for lo, hi in kr]
    mask = []
    for I, (qlo, qhi) in enumerate(qr):
        if pama:
            P = brute_pama(q, kbar, qlo, qhi, scale)
            top = max(P)
            r = [x / top for x in P] if tau_mode == 0 else P
        else:
            s = [scale * _dot(qbar[I], kbar[J]) for J in range(len(kr))]
            top = max(s)
            if tau_mode == 0:        # relative to the row's largest proxy probability
                r = [math.exp(x - top) for x in s]
            else:                    # the proxy probability itself
                z = math.fsum(math.exp(x - top) for x in s)
                r = [math.exp(x - top) / z for x in s]
        ranking = sorted(range(len(kr)), key=lambda J: (-r[J], J))
        if tau_mode == 2:        # shortest ranking prefix with mass >= 1 - tau
            cands = []
            for J in ranking:
                if math.fsum(r[x] for x in cands) >= 1.0 - tau:
                    break
                cands.append(J)
        else:
            cands = [J for J in ranking if r[J] >= tau]
        if max_keep > 0 and len(cands) > max_keep:
            chosen = set(cands[:max_keep])
        elif len(cands) < min_keep:
            chosen = set(ranking[:min_keep])
        else:
            chosen = set(cands)
        row = []
        for J, (klo, _) in enumerate(kr):
            row.append(J in chosen or klo < n_prefix or qlo < n_prefix)
        mask.append(row)
    return mask


def brute_forward(q, k, v, mask, block_q, block_k, scale):
    """(O, LSE) under a given mask, one scalar loop per query row."""
    N, d = len(q), len(q[0])
    qr = _block_ranges(N, block_q)
    kr = _block_ranges(N, block_k)
    kbar = [_mean_rows(k, lo, hi) for lo, hi in kr]
    vbar = [_mean_rows(v, lo, hi) for lo, hi in kr]
    O, LSE = [], []
    for I, (qlo, qhi) in enumerate(qr):
        for i in range(qlo, qhi):
            logits, values = [], []
            for J, (klo, khi) in enumerate(kr):
                if mask[I][J]:
                    for t in range(klo, khi):
                        logits.append(scale * _dot(q[i], k[t]))
                        values.append(v[t])
                else:
                    logits.append(scale * _dot(q[i], kbar[J]) + math.log(khi - klo))
                    values.append(vbar[J])
            M = max(logits)
            w = [math.exp(x - M) for x in logits]
            Z = math.fsum(w)
            O.append([math.fsum(w[j] * values[j][c] for j in range(len(w))) / Z for c in range(d)])
            LSE.append(M + math.log(Z))
    return O, LSE


def brute_dense(q, k, v, scale):
    """Plain softmax attention, scalar loops."""
    N, d = len(q), len(q[0])
    O, LSE = [], []
    for i in range(N):
        logits = [scale * _dot(q[i], k[t]) for t in range(N)]
        M = max(logits)
        w = [math.exp(x - M) for x in logits]
        Z = math.fsum(w)
        O.append([math.fsum(w[t] * v[t][c] for t in range(N)) / Z for c in range(d)])
        LSE.append(M + math.log(Z))
    return O, LSE
