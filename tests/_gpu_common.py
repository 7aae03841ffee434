"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding
and compare it with the CPU oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import sparse_attn_ref as R
from workloads import synth as S

REL_FRO = 1e-2       # output tolerance at bf16 inputs: relative Frobenius error
MAX_ABS = 3e-2       # and max-abs error


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sa():
    import free_block_sparse_route_amd as m
    return m


def cfg_for(w: S.Workload, tau=None, mode=R.RELATIVE, max_keep=None, min_keep=1, prefix=None, no_residual=False,
            proxy=R.CENTROID, fused=False):
    m = sa()
    return m.Config(block_q=w.block_q, block_k=w.block_k, tau=w.tau if tau is None else tau, tau_mode=mode,
                    max_keep=w.max_keep if max_keep is None else max_keep, min_keep=min_keep,
                    n_dense_prefix=w.n_text if prefix is None else prefix, no_residual=no_residual, proxy=proxy,
                    fused=fused)


def oracle_params(cfg) -> R.RouteParams:
    return R.RouteParams(cfg.block_q, cfg.block_k, float(np.float32(cfg.tau)), cfg.tau_mode, cfg.max_keep,
                         cfg.min_keep, cfg.n_dense_prefix, cfg.scale, proxy=cfg.proxy)


def run_gpu(Q, K, V, cfg):
    """Route and forward; O starts as NaN, so that a row no work item wrote (a
    work order or workgroup mapping that skips an item) fails every check."""
    m = sa()
    rt = m.route(Q, K, V, cfg)
    O = torch.full_like(Q, float("nan"))
    O, L = m.forward(Q, K, V, rt, cfg, out=O, lse=True)
    torch.cuda.synchronize()
    return rt, O, L


def head_np(T: torch.Tensor, b: int, h: int) -> np.ndarray:
    return T[b, h].double().cpu().numpy()


def check_lists(rt, lists: bool = True) -> np.ndarray:
    """kv_count, kv_idx (unless fused routing, which writes no lists) and the bit
    mask agree; returns the mask as numpy bool."""
    mask = rt.mask().cpu().numpy()
    cnt = rt.kv_count.cpu().numpy()
    idx = rt.kv_idx.cpu().numpy()
    assert np.array_equal(cnt, mask.sum(axis=-1)), "kv_count != popcount(mask)"
    B, H, n_qb, n_kb = mask.shape
    for b in range(B if lists else 0):
        for h in range(H):
            for I in range(n_qb):
                c = cnt[b, h, I]
                assert np.array_equal(idx[b, h, I, :c], np.flatnonzero(mask[b, h, I])), (b, h, I)
    # bits past n_kb in the last word are zero
    words = rt.kv_mask.cpu().numpy().view(np.uint32)
    tail = rt.n_kb % 32
    if tail:
        assert (words[..., -1] >> np.uint32(tail) == 0).all()
    return mask


def check_mask_head(gpu_mask: np.ndarray, q: np.ndarray, k: np.ndarray, cfg, row_stats=None):
    """Bit-exact outside the rounding band; returns (oracle route, n_diff, n_exempt)."""
    p = oracle_params(cfg)
    rt = R.route_ref(q, k, p)
    diff = gpu_mask != rt.mask
    bad = diff & ~rt.exempt
    assert not bad.any(), f"{int(bad.sum())} mask bits differ outside the 1e-4 band, first {np.argwhere(bad)[:5]}"
    if row_stats is not None:
        np.testing.assert_allclose(row_stats[:, 0], rt.row_max, rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(row_stats[:, 1], rt.row_lse, rtol=1e-5, atol=1e-4)
    return rt, int(diff.sum()), int(rt.exempt.sum())


HEAD_ORDER_MIN_ITEMS = 16 * 768     # work lists of HEAD_ORDER_MIN_ITEMS..HEAD_ORDER_MAX_ITEMS items are
HEAD_ORDER_MAX_ITEMS = 48 * 1024    # ordered head-major
HEAD_ORDER_MAX_NQB = 32 * 64
HEAD_ORDER_MAX_BH = 1024


def expected_work_order(cost: np.ndarray, BH: int, n_qb: int) -> np.ndarray:
    """The forward's work order as the route defines it from the costs: items by cost
    band floor(log2 cost), highest band first, then ascending item; a long list
    (HEAD_ORDER_MIN_ITEMS to HEAD_ORDER_MAX_ITEMS items) head-major instead: heads by total cost
    (highest first, lower head on ties), then band (highest first), then query block."""
    cost = np.asarray(cost).ravel().astype(np.int64)
    item = np.arange(cost.size)
    band = np.floor(np.log2(np.maximum(cost, 1))).astype(np.int64)
    if (HEAD_ORDER_MIN_ITEMS <= cost.size <= HEAD_ORDER_MAX_ITEMS and n_qb <= HEAD_ORDER_MAX_NQB
            and BH <= HEAD_ORDER_MAX_BH):
        hcost = cost.reshape(BH, n_qb).sum(axis=1)
        hrank = np.empty(BH, dtype=np.int64)
        hrank[np.lexsort((np.arange(BH), -hcost))] = np.arange(BH)
        return np.lexsort((item, -band, hrank[item // n_qb]))
    return np.lexsort((item, -band))


def check_work_order(rt):
    """The route's work order equals the one its costs define."""
    cost = rt.cost.cpu().numpy()
    B, H, n_qb = cost.shape
    want = expected_work_order(cost, B * H, n_qb)
    assert np.array_equal(rt.work_order.cpu().numpy(), want), "work order differs from the cost-defined order"


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (8 significant bits): the most that
    rounding a result to a bf16 output moves it."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))   # |x| in [2^(e-1), 2^e)
    return np.ldexp(1.0, e - 9)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_out_head(O_gpu: np.ndarray, L_gpu: np.ndarray, q, k, v, mask, cfg, blocks=None, residual=True):
    """O within REL_FRO / MAX_ABS of the oracle under the given mask (on the listed query blocks)."""
    p = oracle_params(cfg)
    O_ref, L_ref = R.forward_ref_with_mask(q, k, v, mask, p, rows=blocks, residual=residual)
    sel = ~np.isnan(L_ref)
    e_rel = rel_fro(O_gpu[sel], O_ref[sel])
    e_abs = float(np.abs(O_gpu[sel] - O_ref[sel]).max())
    assert e_rel <= REL_FRO and e_abs <= MAX_ABS, f"rel-Frobenius {e_rel:.3e}, max-abs {e_abs:.3e}"
    if L_gpu is not None:
        e_l = float(np.abs(L_gpu[sel] - L_ref[sel]).max())
        assert e_l <= 2e-2, f"LSE max-abs {e_l:.3e}"
    return e_rel, e_abs


def sample_blocks(mask_h: np.ndarray, n_random: int, seed: int) -> list:
    """Query blocks to evaluate in the oracle: first, tail, most and fewest kept, random."""
    n_qb = mask_h.shape[0]
    cnt = mask_h.sum(axis=1)
    rng = np.random.default_rng(seed)
    s = {0, n_qb - 1, int(cnt.argmax()), int(cnt.argmin())}
    s |= set(rng.choice(n_qb, size=min(n_random, n_qb), replace=False).tolist())
    return sorted(s)
