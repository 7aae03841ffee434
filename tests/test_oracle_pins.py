"""Pins of the CPU oracle against facts that do not come from the oracle itself.

  hand       a routing + residual example worked by hand (tests/golden/hand_d1_n4.json)
  (a)        tau = 0 keeps every block, so the result is dense softmax attention:
             torch's scaled_dot_product_attention in float64 and a scalar-loop dense
  (b)        when every key of a block equals the block mean, the residual is exact:
             result == dense attention for every tau and both threshold readings
  (c)        all softmax weights, residual mass included, sum to 1 per row
  (d)        the scalar brute-force oracle agrees to ~1e-12 on tiny inputs
  cap        the top-k budget keeps the max_keep candidates of largest r (subset
             enumeration)
  ABSOLUTE   at most floor(1/tau) blocks clear tau (proxy probabilities sum to 1)
  RELATIVE   the block of largest proxy probability is always kept
  Jensen     block mean key underestimates the block's log-mass, so LSE_sparse <=
             LSE_dense on every row (PARK page, appendix D.2)
  variance   that underestimate is, to leading order, half the within-block
             variance of the scaled scores (PARK page, appendix D.2)
  shift      K + 1c^T leaves mask and output unchanged; V + 1c^T adds c to output
             (a common additive offset does not change a softmax, PARK page, appendix A)
  closed     every block dropped: attention over block-mean keys/values with a
             ln(block size) bias, via torch's SDPA with an additive mask
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute as BR
from oracle import sparse_attn_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(N, d, seed, qs=1.0, ks=1.0):
    rng = np.random.default_rng(seed)
    return (qs * rng.standard_normal((N, d)), ks * rng.standard_normal((N, d)),
            rng.standard_normal((N, d)))


def structured_qkv(N, d, seed, qs=3.0, ks=1.0, period=24):
    """Random q, k with a smooth positional component, so block means differ and
    routing drops blocks; v standard normal."""
    rng = np.random.default_rng(seed)
    pos = np.arange(N)[:, None] * (2 * np.pi / period) * (1 + np.arange(d)[None, :] % 3)
    base = np.sin(pos + rng.uniform(0, 2 * np.pi, d)[None, :])
    q = qs * (base + 0.3 * rng.standard_normal((N, d)))
    k = ks * (base + 0.3 * rng.standard_normal((N, d)))
    return q, k, rng.standard_normal((N, d))


def sdpa64(q, k, v, scale, bias=None):
    """torch's scaled_dot_product_attention in float64 on CPU (math backend)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).double()[None, None] for x in (q, k, v))
    mask = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).double()[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    return o[0, 0].numpy()


def lse_dense(q, k, scale):
    S = scale * (q @ k.T)
    m = S.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]


SHAPES = [  # N, d, bq, bk, prefix
    (1, 4, 4, 4, 0), (7, 4, 4, 2, 0), (7, 4, 2, 4, 3), (64, 4, 8, 16, 0), (64, 8, 16, 8, 16),
    (257, 16, 64, 64, 0), (257, 64, 128, 64, 0), (257, 64, 64, 128, 130), (200, 8, 32, 16, 0),
]


# ----------------------------------------------------------------------------- hand
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_d1_n4.json")))
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    for case in g["cases"]:
        p = R.RouteParams(g["block_q"], g["block_k"], case["tau"], case["tau_mode"], scale=g["scale"])
        O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
        assert rt.mask.tolist() == case["mask"]
        np.testing.assert_allclose(O, np.array(case["O"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(L, np.array(case["LSE"]), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- (a)
@pytest.mark.parametrize("N,d,bq,bk,prefix", SHAPES)
@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE])
def test_a_tau_zero_is_dense(N, d, bq, bk, prefix, mode):
    q, k, v = rand_qkv(N, d, 1000 + N + d, qs=3.0)
    p = R.RouteParams(bq, bk, 0.0, mode, n_prefix=prefix)
    O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
    assert rt.mask.all()
    sig = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(O, sdpa64(q, k, v, sig), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, lse_dense(q, k, sig), rtol=0, atol=1e-12)
    Od, Ld = R.dense_ref(q, k, v)
    np.testing.assert_allclose(Od, sdpa64(q, k, v, sig), rtol=0, atol=1e-12)
    if N <= 64:
        Ob, Lb = BR.brute_dense(q.tolist(), k.tolist(), v.tolist(), sig)
        np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- (b)
@pytest.mark.parametrize("N,d,bq,bk,prefix", SHAPES)
@pytest.mark.parametrize("mode,tau", [(R.RELATIVE, 0.05), (R.RELATIVE, 0.5), (R.ABSOLUTE, 0.02),
                                      (R.ABSOLUTE, 2.0)])
def test_b_identical_keys_make_residual_exact(N, d, bq, bk, prefix, mode, tau):
    rng = np.random.default_rng(7 + N)
    n_kb = -(-N // bk)
    per_block = 2.0 * rng.standard_normal((n_kb, d))
    k = np.repeat(per_block, bk, axis=0)[:N]              # every key of block J is the same
    q = 3.0 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    p = R.RouteParams(bq, bk, tau, mode, n_prefix=prefix, min_keep=0 if tau > 1 else 1)
    O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
    sig = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(O, sdpa64(q, k, v, sig), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, lse_dense(q, k, sig), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- (c)
@pytest.mark.parametrize("N,d,bq,bk,prefix", SHAPES)
def test_c_weights_sum_to_one(N, d, bq, bk, prefix):
    q, k, v = rand_qkv(N, d, 55 + N, qs=4.0)
    p = R.RouteParams(bq, bk, 0.2, R.RELATIVE, n_prefix=prefix)
    rt = R.route_ref(q, k, p)
    _, _, W = R.forward_ref_with_mask(q, k, v, rt.mask, p, return_weights=True)
    for tok, wt, dropped, wb in W:
        assert (wt >= 0).all() and (wb >= 0).all()
        tot = wt.sum(axis=1) + wb.sum(axis=1)
        np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)
        # each row weighs every token of the sequence exactly once: kept tokens one by
        # one, dropped blocks as a whole
        n_j = R.block_counts(N, bk)
        assert len(tok) + n_j[dropped].sum() == N


# ----------------------------------------------------------------------------- (d)
BRUTE = [  # N, d, bq, bk, prefix, tau, mode, max_keep, min_keep
    (1, 3, 2, 2, 0, 0.5, 0, 0, 1), (5, 3, 2, 2, 0, 0.3, 0, 0, 1), (9, 4, 4, 2, 0, 0.1, 1, 0, 1),
    (9, 4, 2, 4, 0, 0.2, 0, 2, 1), (16, 4, 4, 4, 5, 0.6, 0, 0, 1), (23, 5, 4, 3, 0, 0.05, 1, 3, 2),
    (31, 3, 8, 4, 0, 1.5, 0, 0, 0), (31, 3, 8, 4, 0, 1.5, 1, 0, 2), (40, 6, 8, 8, 9, 0.02, 1, 2, 1), (40, 6, 8, 4, 16, 0.3, 0, 0, 1),
    (64, 4, 16, 8, 0, 0.01, 0, 4, 1), (64, 4, 8, 16, 0, 0.25, 1, 0, 1), (33, 2, 4, 4, 0, 0.7, 0, 5, 3),
    # TOPP: shortest ranking prefix with proxy mass >= 1 - tau
    (40, 6, 8, 4, 0, 0.1, 2, 0, 1), (64, 4, 8, 8, 0, 0.3, 2, 3, 1), (33, 5, 4, 4, 9, 0.05, 2, 0, 2),
    (31, 3, 8, 4, 0, 1.0, 2, 0, 0), (23, 4, 4, 2, 0, 0.0, 2, 0, 1),
]


@pytest.mark.parametrize("N,d,bq,bk,prefix,tau,mode,mk,mn", BRUTE)
def test_d_brute_force_agrees(N, d, bq, bk, prefix, tau, mode, mk, mn):
    q, k, v = rand_qkv(N, d, 31 * N + d, qs=2.5)
    sig = 1.0 / math.sqrt(d)
    p = R.RouteParams(bq, bk, tau, mode, max_keep=mk, min_keep=mn, n_prefix=prefix)
    O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
    bm = BR.brute_route(q.tolist(), k.tolist(), bq, bk, tau, mode, mk, mn, prefix, sig)
    assert np.array_equal(rt.mask, np.array(bm, dtype=bool))
    Ob, Lb = BR.brute_forward(q.tolist(), k.tolist(), v.tolist(), bm, bq, bk, sig)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


def test_d_brute_force_covers_drops():
    """The brute-force cases exercise dropped blocks (otherwise (d) would only test dense)."""
    dropped = 0
    for N, d, bq, bk, prefix, tau, mode, mk, mn in BRUTE:
        q, k, v = rand_qkv(N, d, 31 * N + d, qs=2.5)
        rt = R.route_ref(q, k, R.RouteParams(bq, bk, tau, mode, max_keep=mk, min_keep=mn,
                                             n_prefix=prefix))
        dropped += int((~rt.mask).sum())
    assert dropped > 20


# ----------------------------------------------------------------------------- cap
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE])
def test_cap_is_best_subset(seed, mode):
    N, d, bq, bk = 80, 8, 8, 8                       # n_kb = 10
    q, k, v = rand_qkv(N, d, 900 + seed, qs=2.0)
    mk = 3
    tau = 0.05 if mode == R.RELATIVE else 0.02
    p = R.RouteParams(bq, bk, tau, mode, max_keep=mk, min_keep=0)
    rt = R.route_ref(q, k, p)
    binding = 0
    for I in range(rt.mask.shape[0]):
        r = rt.r[I]
        C = [J for J in range(len(r)) if r[J] >= tau]
        kept = set(np.flatnonzero(rt.mask[I]).tolist())
        if len(C) <= mk:
            assert kept == set(C)
            continue
        binding += 1
        best = max(itertools.combinations(C, mk), key=lambda S: (sum(r[j] for j in S), [-j for j in S]))
        assert kept == set(best)
    assert binding > 0


def test_cap_tie_break_prefers_lower_block_index():
    """Exact ties in r (identical key blocks) are broken by key-block index, ascending."""
    rng = np.random.default_rng(8)
    d, bk = 8, 8
    blk = rng.standard_normal((bk, d))
    k = np.concatenate([blk] * 6)                    # six identical key blocks: r ties exactly
    q, _, v = rand_qkv(48, d, 9, qs=2.0)
    for mode in (R.RELATIVE, R.ABSOLUTE):
        p = R.RouteParams(16, bk, 0.0, mode, max_keep=2, min_keep=0)
        rt = R.route_ref(q, k, p)
        assert (rt.mask == np.array([True, True, False, False, False, False])).all()
        bm = BR.brute_route(q.tolist(), k.tolist(), 16, bk, 0.0, mode, 2, 0, 0, 1 / math.sqrt(d))
        assert np.array_equal(rt.mask, np.array(bm, dtype=bool))
    # floor: nothing clears tau > 1, the first min_keep of the ranking are kept
    p = R.RouteParams(16, bk, 2.0, R.RELATIVE, min_keep=3)
    assert (R.route_ref(q, k, p).mask == np.array([True] * 3 + [False] * 3)).all()


# ----------------------------------------------------------------------------- thresholds
@pytest.mark.parametrize("tau", [0.5, 0.2, 0.05, 0.01])
def test_absolute_keeps_at_most_inverse_tau(tau):
    q, k, v = rand_qkv(4096, 16, 3, qs=0.3)          # flat proxy rows: many blocks near 1/n_kb
    p = R.RouteParams(64, 32, tau, R.ABSOLUTE, min_keep=0)
    rt = R.route_ref(q, k, p)
    assert rt.mask.sum(axis=1).max() <= math.floor(1.0 / tau)
    # the bound is tight enough to matter: the flat rows would otherwise keep more
    p_rel = R.RouteParams(64, 32, tau, R.RELATIVE, min_keep=0)
    assert R.route_ref(q, k, p_rel).mask.sum(axis=1).max() > math.floor(1.0 / tau)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("tau", [0.05, 0.3, 0.7])
def test_topp_is_smallest_set_reaching_the_mass(seed, tau):
    """TOPP keeps a minimum-cardinality set of key blocks whose proxy mass reaches
    1 - tau (found by enumerating subsets), and of those the one of largest mass."""
    N, d, bq, bk = 80, 8, 8, 8                       # n_kb = 10
    q, k, v = rand_qkv(N, d, 700 + seed, qs=2.0)
    p = R.RouteParams(bq, bk, tau, R.TOPP, min_keep=0)
    rt = R.route_ref(q, k, p)
    for I in range(rt.mask.shape[0]):
        P = rt.r[I]
        assert abs(P.sum() - 1.0) < 1e-12
        kept = set(np.flatnonzero(rt.mask[I]).tolist())
        size = next(n for n in range(len(P) + 1)
                    if any(sum(P[j] for j in S) >= 1 - tau for S in itertools.combinations(range(len(P)), n)))
        assert len(kept) == size
        best = max(itertools.combinations(range(len(P)), size), key=lambda S: (sum(P[j] for j in S), [-j for j in S]))
        assert kept == set(best)


def test_topp_tau_zero_is_dense():
    """TOPP with tau = 0 needs the whole proxy mass: every block is kept (no proxy
    probability underflows at this scale) and the output is dense attention."""
    q, k, v = rand_qkv(96, 8, 21, qs=1.0)
    p = R.RouteParams(16, 8, 0.0, R.TOPP)
    rt = R.route_ref(q, k, p)
    assert rt.mask.all()
    O, L = R.forward_ref(q, k, v, p)
    Od, Ld = R.dense_ref(q, k, v)
    assert np.abs(O - Od).max() < 1e-12 and np.abs(L - Ld).max() < 1e-12


@pytest.mark.parametrize("tau", [1.0, 0.5, 0.01])
def test_relative_always_keeps_argmax(tau):
    q, k, v = rand_qkv(1000, 8, 11, qs=5.0)
    p = R.RouteParams(50, 40, tau, R.RELATIVE, min_keep=0)
    rt = R.route_ref(q, k, p)
    arg = rt.s.argmax(axis=1)
    assert rt.mask[np.arange(len(arg)), arg].all()


def test_prefix_rows_and_columns_dense():
    q, k, v = rand_qkv(300, 8, 12, qs=5.0)
    p = R.RouteParams(32, 16, 0.9, R.RELATIVE, n_prefix=40)
    rt = R.route_ref(q, k, p)
    assert rt.mask[:, :3].all()                      # key blocks starting at 0, 16, 32 < 40
    assert rt.mask[:2].all()                         # query blocks starting at 0, 32 < 40
    assert not rt.mask[2:, 3:].all()


# ----------------------------------------------------------------------------- Jensen / variance
@pytest.mark.parametrize("seed", range(4))
def test_jensen_sparse_lse_below_dense(seed):
    q, k, v = structured_qkv(500, 16, 77 + seed, period=200)
    p = R.RouteParams(64, 32, 0.3, R.RELATIVE)
    O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
    assert (~rt.mask).sum() > 0
    Ld = lse_dense(q, k, 1.0 / 4.0)
    assert (L <= Ld + 1e-12).all()
    assert (L < Ld - 1e-6).any()


def test_half_variance_leading_error():
    rng = np.random.default_rng(5)
    n, d = 16, 8
    q = rng.standard_normal((1, d))
    kbar = rng.standard_normal(d)
    u = rng.standard_normal((n, d))
    u -= u.mean(axis=0)                              # deviations sum to zero
    v = rng.standard_normal((n, d))
    sig = 1.0 / math.sqrt(d)
    for eps in (1e-2, 3e-3, 1e-3):
        k = kbar + eps * u
        qq = np.repeat(q, n, axis=0)                 # one query block of identical rows
        p = R.RouteParams(n, n, 2.0, R.RELATIVE, min_keep=0)     # tau > 1: drop everything
        _, L = R.forward_ref(qq, k, v, p)
        x = sig * (k @ q[0])
        gap = lse_dense(qq[:1], k, sig)[0] - L[0]
        ratio = gap / (0.5 * x.var())
        assert abs(ratio - 1.0) < 1e-3 * (eps / 1e-3) + 1e-4, (eps, ratio)


# ----------------------------------------------------------------------------- shift
@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE])
def test_key_shift_invariance(mode):
    q, k, v = rand_qkv(333, 16, 21, qs=3.0)
    c = np.random.default_rng(2).standard_normal(16) * 2.0
    p = R.RouteParams(32, 64, 0.1 if mode == R.RELATIVE else 0.03, mode)
    O1, L1, r1 = R.forward_ref(q, k, v, p, return_route=True)
    O2, L2, r2 = R.forward_ref(q, k + c, v, p, return_route=True)
    diff = r1.mask != r2.mask
    assert not (diff & ~r1.exempt).any()
    if not diff.any():
        np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-10)


def test_value_shift_adds_constant():
    q, k, v = rand_qkv(333, 16, 22, qs=3.0)
    c = np.random.default_rng(3).standard_normal(16)
    p = R.RouteParams(32, 64, 0.1, R.RELATIVE)
    O1, _ = R.forward_ref(q, k, v, p)
    O2, _ = R.forward_ref(q, k, v + c, p)
    np.testing.assert_allclose(O2, O1 + c, rtol=0, atol=1e-12)


def test_within_block_permutation_invariance():
    N, bk = 256, 32
    q, k, v = rand_qkv(N, 8, 23, qs=3.0)
    rng = np.random.default_rng(4)
    perm = np.concatenate([J * bk + rng.permutation(bk) for J in range(N // bk)])
    p = R.RouteParams(64, bk, 0.2, R.RELATIVE)
    O1, L1 = R.forward_ref(q, k, v, p)
    O2, L2 = R.forward_ref(q, k[perm], v[perm], p)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- closed form
@pytest.mark.parametrize("N,bk", [(100, 16), (256, 64), (257, 128)])
def test_all_dropped_closed_form(N, bk):
    d = 16
    q, k, v = rand_qkv(N, d, 41 + N, qs=2.0)
    p = R.RouteParams(32, bk, 5.0, R.ABSOLUTE, min_keep=0)
    O, L, rt = R.forward_ref(q, k, v, p, return_route=True)
    assert not rt.mask.any()
    tk = torch.from_numpy(k)
    tv = torch.from_numpy(v)
    n_kb = -(-N // bk)
    kb = torch.stack([tk[J * bk:(J + 1) * bk].mean(0) for J in range(n_kb)]).numpy()
    vb = torch.stack([tv[J * bk:(J + 1) * bk].mean(0) for J in range(n_kb)]).numpy()
    sizes = np.array([min((J + 1) * bk, N) - J * bk for J in range(n_kb)], dtype=np.float64)
    bias = np.broadcast_to(np.log(sizes)[None, :], (N, n_kb))
    np.testing.assert_allclose(O, sdpa64(q, kb, vb, 1.0 / 4.0, bias=bias), rtol=0, atol=1e-12)


def test_no_residual_is_attention_over_kept_tokens():
    """Without the residual, each query block attends to exactly its kept tokens: compare
    with torch SDPA over the gathered kept keys and values."""
    q, k, v = structured_qkv(300, 8, 31, period=150)
    p = R.RouteParams(32, 16, 0.4, R.RELATIVE)
    rt = R.route_ref(q, k, p)
    O, L = R.forward_ref_with_mask(q, k, v, rt.mask, p, residual=False)
    assert (~rt.mask).any()
    for I in range(rt.mask.shape[0]):
        tok = np.concatenate([np.arange(J * 16, min(J * 16 + 16, 300)) for J in np.flatnonzero(rt.mask[I])])
        rows = slice(I * 32, min(I * 32 + 32, 300))
        np.testing.assert_allclose(O[rows], sdpa64(q[rows], k[tok], v[tok], 1 / math.sqrt(8)), rtol=0, atol=1e-12)


def test_recall_is_one_when_all_kept():
    q, k, v = rand_qkv(128, 8, 9)
    p = R.RouteParams(32, 32, 0.0)
    rt = R.route_ref(q, k, p)
    assert abs(R.attention_recall(q, k, rt.mask, p) - 1.0) < 1e-12


def test_recall_hand_worked_partial_mask():
    """Attention recall (PARK page, section 3.2: the share of the dense softmax
    weight that lands in retained blocks, averaged over queries) worked by hand
    on d = 1, N = 4 with a logit scale of 1/2 and block 0 dropped for both
    query blocks.

    q = (1, 1, 0, 0), k = (-1, 1, 2, 0): the rows with q = 1 have logits
    (-1/2, 1/2, 1, 0) and keep tokens 2, 3, so their recall is
    (e + 1) / (e^(-1/2) + e^(1/2) + e + 1); the rows with q = 0 weigh all four
    keys equally and keep two of them, recall 1/2.  A dropped scale (logits
    -1, 1, 2, 0) or a mask indexed [key block, query block] (which would drop
    tokens 2, 3 of the first rows and keep all of the last) give other values;
    block_q = 4 (one query block) with block_k = 2 gives the same value."""
    q = np.array([[1.0], [1.0], [0.0], [0.0]])
    k = np.array([[-1.0], [1.0], [2.0], [0.0]])
    e = math.e
    first = (e + 1.0) / (math.exp(-0.5) + math.exp(0.5) + e + 1.0)
    want = (2.0 * first + 2.0 * 0.5) / 4.0
    p = R.RouteParams(2, 2, 0.0, scale=0.5)
    mask = np.array([[False, True], [False, True]])
    assert abs(R.attention_recall(q, k, mask, p) - want) < 1e-12
    p1 = R.RouteParams(4, 2, 0.0, scale=0.5)
    assert abs(R.attention_recall(q, k, np.array([[False, True]]), p1) - want) < 1e-12
    # the two plausible mistakes give different numbers
    unscaled = (2.0 * (e * e + 1.0) / (math.exp(-1.0) + e + e * e + 1.0) + 1.0) / 4.0
    transposed = (2.0 * 0.0 + 2.0 * 1.0) / 4.0
    assert abs(want - unscaled) > 1e-2 and abs(want - transposed) > 1e-2


# ----------------------------------------------------------------------------- PAMA proxy
# Per-query attention-mass aggregation (PARK page, section 5.1): each query's
# softmax over the key-block means, averaged within its query block.
PAMA_BRUTE = [  # N, d, bq, bk, prefix, tau, mode, max_keep, min_keep
    (40, 6, 8, 4, 0, 0.1, 0, 0, 1), (40, 6, 8, 4, 0, 0.05, 1, 0, 1), (40, 6, 8, 4, 0, 0.1, 2, 0, 1),
    (33, 5, 4, 4, 9, 0.2, 0, 3, 2), (31, 3, 8, 4, 0, 0.3, 2, 2, 1), (23, 4, 4, 2, 0, 0.0, 1, 0, 1),
]


@pytest.mark.parametrize("N,d,bq,bk,prefix,tau,mode,mk,mn", PAMA_BRUTE)
def test_pama_brute_force_agrees(N, d, bq, bk, prefix, tau, mode, mk, mn):
    q, k, v = rand_qkv(N, d, 7 * N + d, qs=2.5)
    sig = 1.0 / math.sqrt(d)
    p = R.RouteParams(bq, bk, tau, mode, max_keep=mk, min_keep=mn, n_prefix=prefix, proxy=R.PAMA)
    rt = R.route_ref(q, k, p)
    bm = BR.brute_route(q.tolist(), k.tolist(), bq, bk, tau, mode, mk, mn, prefix, sig, pama=True)
    assert np.array_equal(rt.mask, np.array(bm, dtype=bool))
    kbar = R.pool(k, bk)
    for I in range(R.n_blocks(N, bq)):
        want = BR.brute_pama(q.tolist(), kbar.tolist(), I * bq, min((I + 1) * bq, N), sig)
        np.testing.assert_allclose(np.exp(rt.s[I]), want, rtol=0, atol=1e-13)


def test_pama_rows_are_distributions():
    q, k, _ = rand_qkv(100, 8, 5, qs=3.0)
    A = R.pama_importance(q, R.pool(k, 16), 32, 1 / math.sqrt(8))
    assert A.shape == (4, 7) and (A > 0).all()
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE, R.TOPP])
def test_pama_equals_centroid_proxy_for_identical_queries(mode):
    """When every query of a block is the same vector, averaging after the
    softmax equals the softmax of the mean query: PAMA reduces to the centroid
    proxy, decisions and scores alike."""
    rng = np.random.default_rng(11)
    bq, N, d = 8, 48, 6
    q = np.repeat(rng.standard_normal((N // bq, d)) * 3, bq, axis=0)
    k = rng.standard_normal((N, d))
    pc = R.RouteParams(bq, 4, 0.05, mode)
    pp = R.RouteParams(bq, 4, 0.05, mode, proxy=R.PAMA)
    rc, rp = R.route_ref(q, k, pc), R.route_ref(q, k, pp)
    np.testing.assert_allclose(rp.r, rc.r, rtol=0, atol=1e-13)
    assert np.array_equal(rp.mask, rc.mask)


def test_pama_keeps_what_query_averaging_erases():
    """Two opposite queries in one block and key-block means +e, -e, 0: the mean
    query is 0, so the centroid proxy is uniform, while each query's own softmax
    peaks on one of the first two blocks.  Closed form with a = sigma c:
    A = (cosh a, cosh a, 1) / (2 cosh a + 1)."""
    d, c = 4, 6.0
    e = np.zeros(d); e[0] = 1.0
    q = np.stack([c * e, -c * e])
    k = np.stack([e, e, -e, -e, 0 * e, 0 * e])             # block size 2: means +e, -e, 0
    sig = 1 / math.sqrt(d)
    a = sig * c
    want = np.array([math.cosh(a), math.cosh(a), 1.0]) / (2 * math.cosh(a) + 1)
    A = R.pama_importance(q, R.pool(k, 2), 2, sig)
    np.testing.assert_allclose(A[0], want, rtol=1e-14)
    pp = R.RouteParams(2, 2, 0.5, R.RELATIVE, proxy=R.PAMA)
    pc = R.RouteParams(2, 2, 0.5, R.RELATIVE)
    assert R.route_ref(q, k, pp).mask[0].tolist() == [True, True, False]
    assert R.route_ref(q, k, pc).mask[0].tolist() == [True, True, True]
