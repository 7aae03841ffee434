"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the whole workload runs on the GPU; masks are checked against the
oracle on every head (Wan-1.3B) or on sampled heads, outputs on sampled query
blocks (first, tail, most- and fewest-kept, random), and list/mask consistency
and finiteness on everything."""
import numpy as np
import pytest
import torch

from oracle import sparse_attn_ref as R
from workloads import synth as S

from _gpu_common import (check_lists, check_mask_head, check_out_head, check_work_order, cfg_for, head_np, run_gpu,
                         sample_blocks, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def check_workload(w, cfgs, heads, blocks_per_head=6, lists=True):
    say(f"[case] {w.name}: generating B{w.B} H{w.H} N{w.N}")
    Qc, Kc, Vc = S.make_qkv(w)
    Q, K, V = Qc.cuda(), Kc.cuda(), Vc.cuda()
    for cfg in cfgs:
        say(f"[case] {w.name} tau={cfg.tau} mode={cfg.tau_mode} cap={cfg.max_keep} prefix={cfg.n_dense_prefix}")
        rt, O, L = run_gpu(Q, K, V, cfg)
        mask = check_lists(rt, lists=lists)
        check_work_order(rt)
        stats = rt.row_stats.cpu().numpy()
        assert torch.isfinite(O).all().item() and torch.isfinite(L).all().item()
        nd_tot = 0
        for b, h in heads:
            q, k, v = head_np(Qc, b, h), head_np(Kc, b, h), head_np(Vc, b, h)
            ort, nd, ne = check_mask_head(mask[b, h], q, k, cfg, stats[b, h])
            nd_tot += nd
            blocks = sample_blocks(mask[b, h], blocks_per_head, 31 * h + b)
            o = O[b, h].float().cpu().numpy()
            l = L[b, h].cpu().numpy()
            e_rel, e_abs = check_out_head(o, l, q, k, v, mask[b, h], cfg, blocks=blocks)
            say(f"   b{b} h{h}: kept {mask[b, h].mean():.4f} band bits differing {nd}/{ne} "
                f"rel-fro {e_rel:.2e} max-abs {e_abs:.2e}")
        say(f"  kept fraction {mask.mean():.4f}; differing band bits on checked heads {nd_tot}")
    del Q, K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE, R.TOPP])
def test_wan13b_full(mode):
    w = S.WORKLOADS["wan1.3b"]
    # TOPP retains 1 - tau of the proxy mass: tau = 0.1 here (0.01 would keep ~95%)
    cfg = cfg_for(w, mode=mode, tau=0.1 if mode == R.TOPP else None)
    check_workload(w, [cfg], [(0, h) for h in range(w.H)], blocks_per_head=6)


@pytest.mark.parametrize("mode", [R.RELATIVE, R.TOPP])
def test_wan13b_full_pama(mode):
    """PAMA proxy on the full Wan-1.3B shape (PARK retrieves by cumulative
    importance: TOPP at tau 0.1; RELATIVE at the workload's tau)."""
    w = S.WORKLOADS["wan1.3b"]
    cfg = cfg_for(w, mode=mode, tau=0.1 if mode == R.TOPP else None, proxy=R.PAMA)
    check_workload(w, [cfg], heads=[(0, h) for h in range(w.H)])


def test_wan14b_pama():
    """PAMA on the full Wan-14B shape in the benchmark's setting (TOPP at tau 0.1,
    cap of 295 blocks): 1182 key blocks per row, two query blocks per workgroup."""
    w = S.WORKLOADS["wan14b"]
    cfg = cfg_for(w, mode=R.TOPP, tau=0.1, proxy=R.PAMA)
    check_workload(w, [cfg], [(0, 0), (0, 39)], blocks_per_head=3)


def test_pama_rows_past_64k_of_lds():
    """PAMA with 1700 key blocks per row (block_k = 64): its workgroup takes
    more than 64 KB of LDS, which the launch must request explicitly."""
    w = S.small("pama_1700", 1, 1, 128, (17, 80, 80), 128, 64, 0.1, qscale=6.0)
    cfg = cfg_for(w, mode=R.TOPP, tau=0.1, proxy=R.PAMA)
    check_workload(w, [cfg], [(0, 0)], blocks_per_head=3)


def test_wan13b_full_fused():
    """Fused routing (decisions inside the forward) on the full Wan-1.3B shape."""
    w = S.WORKLOADS["wan1.3b"]
    cfg = cfg_for(w, fused=True)
    check_workload(w, [cfg], heads=[(0, h) for h in range(w.H)], lists=False)


def test_wan14b_tau_sweep():
    w = S.WORKLOADS["wan14b"]
    cfgs = [cfg_for(w, tau=t) for t in S.WAN14B_TAU_SWEEP] + [cfg_for(w, tau=0.003, mode=R.ABSOLUTE)]
    check_workload(w, cfgs, [(0, 0), (0, 17), (0, 39)], blocks_per_head=4)


def test_hunyuan():
    w = S.WORKLOADS["hunyuan"]
    check_workload(w, [cfg_for(w)], [(0, 0), (0, 11), (0, 23)], blocks_per_head=4)


def test_stress():
    w = S.WORKLOADS["stress"]
    s = S.query_scales(w)
    heads = [(0, int(s.argmin())), (1, int(s.argmax())), (1, int(np.argsort(s)[len(s) // 2]))]
    check_workload(w, [cfg_for(w)], heads, blocks_per_head=4)


@pytest.mark.parametrize("fused", [False, True], ids=["two_kernel", "fused"])
def test_key_blocks_at_the_limit(fused):
    """The largest key-block count the route accepts (16368 blocks of 64 tokens,
    N = 1047552): one proxy row fills a select workgroup's 64 KB of LDS (one query
    block per workgroup, the row read from LDS), the kept lists run long, and
    fused routing holds 512 decision words per work item."""
    w = S.small("limit", 1, 1, 64, (32, 32, 1023), 128, 64, 0.05, qscale=4.0)
    assert w.n_kb == 16384 - 16                  # the route's key-block limit
    cfg = cfg_for(w, fused=fused)
    check_workload(w, [cfg], [(0, 0)], blocks_per_head=1, lists=not fused)
