"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Masks: bit-exact except blocks whose compared quantity lies within 1e-4 of its
cut (tau, or the budget's cut), which the oracle lists.  Outputs: relative
Frobenius error <= 1e-2 and max-abs error <= 3e-2 against the oracle evaluated
on the GPU's own mask (and on the oracle's mask when they agree).
"""
import numpy as np
import pytest
import torch

from oracle import sparse_attn_ref as R
from workloads import synth as S

from _gpu_common import (check_lists, check_mask_head, check_out_head, check_work_order, cfg_for,
                         expected_work_order, head_np, run_gpu, sa, sample_blocks, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def make(w, heads=None):
    Q, K, V = S.make_qkv(w, heads=heads)
    return Q, K, V, Q.cuda(), K.cuda(), V.cuda()


def full_check(w, cfg, blocks_per_head=None, heads=None, label=""):
    """Run route + forward on the whole workload, then check the listed heads against the oracle."""
    say(f"[case] {label} {w.name} B{w.B} H{w.H} N{w.N} d{w.d} {w.block_q}x{w.block_k} {w.dtype} "
        f"tau={cfg.tau} mode={cfg.tau_mode} cap={cfg.max_keep} floor={cfg.min_keep} prefix={cfg.n_dense_prefix}")
    Qc, Kc, Vc, Q, K, V = make(w)
    rt, O, L = run_gpu(Q, K, V, cfg)
    mask = check_lists(rt, lists=not cfg.fused)
    stats = rt.row_stats.cpu().numpy()
    Oc = O.float().cpu().numpy()
    Lc = L.cpu().numpy()
    assert np.isfinite(Oc).all() and np.isfinite(Lc).all()
    heads = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    tot_diff = tot_exempt = 0
    for b, h in heads:
        q, k, v = head_np(Qc, b, h), head_np(Kc, b, h), head_np(Vc, b, h)
        ort, nd, ne = check_mask_head(mask[b, h], q, k, cfg, stats[b, h])
        tot_diff += nd
        tot_exempt += ne
        blocks = None if blocks_per_head is None else sample_blocks(mask[b, h], blocks_per_head, 17 * h + b)
        check_out_head(Oc[b, h], Lc[b, h], q, k, v, mask[b, h], cfg, blocks=blocks,
                       residual=not cfg.no_residual)
        if nd == 0 and blocks is not None:
            pass  # same mask: the check above is also the check against the oracle's own mask
        elif nd:
            # the oracle's own mask differs only inside the band: outputs still agree
            check_out_head(Oc[b, h], Lc[b, h], q, k, v, ort.mask, cfg, blocks=blocks,
                           residual=not cfg.no_residual)
    say(f"  kept {mask.mean():.4f}  band-exempt bits that differ {tot_diff} (of {tot_exempt} in the band)")
    return rt, O, L, mask


# ----------------------------------------------------------------------------- small cases
SMALL = [
    # name, grid, d, bq, bk, dtype, tau, mode, max_keep, min_keep, n_text, hilbert, B, H
    ("r128", (4, 8, 32), 128, 128, 128, "bf16", 0.01, R.RELATIVE, 0, 1, 0, False, 1, 2),
    ("ragged_cap", (5, 8, 25), 128, 128, 64, "bf16", 0.003, R.RELATIVE, 4, 1, 0, False, 1, 2),
    ("abs", (4, 8, 32), 128, 128, 128, "bf16", 0.02, R.ABSOLUTE, 0, 1, 0, False, 1, 2),
    ("abs_floor", (4, 8, 31), 128, 128, 64, "bf16", 0.5, R.ABSOLUTE, 0, 3, 0, False, 2, 1),
    ("prefix_hilbert", (4, 8, 30), 128, 128, 128, "bf16", 0.01, R.RELATIVE, 0, 1, 100, True, 1, 2),
    ("all_dropped", (3, 8, 27), 128, 128, 128, "bf16", 2.0, R.RELATIVE, 0, 0, 0, False, 1, 1),
    ("f32_d64", (4, 8, 16), 64, 64, 64, "f32", 0.02, R.RELATIVE, 0, 1, 0, False, 1, 2),
    ("f32_d128", (3, 7, 19), 128, 128, 64, "f32", 0.02, R.ABSOLUTE, 3, 1, 0, False, 1, 1),
    ("d64_q128_k64", (3, 9, 21), 64, 128, 64, "bf16", 0.01, R.RELATIVE, 0, 1, 0, False, 1, 2),
    ("d128_q64_k128", (3, 9, 21), 128, 64, 128, "bf16", 0.01, R.RELATIVE, 5, 1, 0, False, 1, 2),
    ("multi_bh", (2, 6, 20), 128, 128, 64, "bf16", 0.02, R.RELATIVE, 0, 1, 0, False, 2, 3),
    ("n1", (1, 1, 1), 128, 128, 128, "bf16", 0.01, R.RELATIVE, 0, 1, 0, False, 1, 1),
    ("n63", (1, 7, 9), 64, 64, 64, "bf16", 0.05, R.RELATIVE, 0, 1, 0, False, 1, 1),
    ("n130", (1, 10, 13), 128, 128, 64, "bf16", 0.05, R.ABSOLUTE, 0, 1, 0, False, 1, 1),
    ("big_prefix", (2, 5, 20), 128, 128, 64, "bf16", 0.03, R.RELATIVE, 2, 1, 300, False, 1, 1),
    ("topp", (4, 8, 32), 128, 128, 64, "bf16", 0.05, R.TOPP, 0, 1, 0, False, 1, 2),
    ("topp_cap_prefix", (3, 8, 27), 128, 128, 128, "bf16", 0.02, R.TOPP, 3, 1, 100, True, 1, 2),
    ("topp_f32_floor", (4, 8, 16), 64, 64, 64, "f32", 0.6, R.TOPP, 0, 2, 0, False, 1, 1),
    ("topp_all", (2, 8, 20), 128, 128, 64, "bf16", 0.0, R.TOPP, 0, 1, 0, False, 1, 1),
    ("topp_none", (2, 8, 20), 128, 128, 64, "bf16", 1.0, R.TOPP, 0, 0, 0, False, 1, 1),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case):
    name, grid, d, bq, bk, dt, tau, mode, mk, mn, n_text, hil, B, H = case
    w = S.small(name, B, H, d, grid, bq, bk, tau, dtype=dt, qscale=6.0, n_text=n_text, hilbert=hil)
    cfg = cfg_for(w, mode=mode, max_keep=mk, min_keep=mn)
    full_check(w, cfg, label="small")


def _random_case(seed):
    """A seeded draw over the configuration space the route and forward accept:
    head size, block sizes, dtype, ragged grids, every tau mode with its range,
    cap, floor, dense prefix, Hilbert order, fused routing, the PAMA proxy, batch
    and heads."""
    rng = np.random.default_rng(np.random.SeedSequence((2026, seed)))
    d = int(rng.choice([64, 128]))
    bq, bk = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    dt = "f32" if rng.random() < 0.2 else "bf16"
    while True:
        grid = (int(rng.integers(1, 6)), int(rng.integers(1, 11)), int(rng.integers(1, 41)))
        if grid[0] * grid[1] * grid[2] <= 4000:
            break
    mode = [R.RELATIVE, R.ABSOLUTE, R.TOPP][int(rng.choice(3, p=[0.5, 0.25, 0.25]))]
    tau = (float(10 ** rng.uniform(-3, -0.5)) if mode == R.RELATIVE else
           float(10 ** rng.uniform(-3, -0.3)) if mode == R.ABSOLUTE else float(rng.uniform(0.0, 0.6)))
    n_text = int(rng.integers(1, 300)) if rng.random() < 0.3 else 0
    hil = bool(rng.random() < 0.3)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    fused = bool(mode != R.TOPP and dt == "bf16" and rng.random() < 0.2)
    N = grid[0] * grid[1] * grid[2] + n_text
    n_kb = -(-N // bk)
    mk = 0 if (fused or rng.random() < 0.6) else int(rng.integers(1, n_kb + 1))
    mn = int(rng.integers(0, 2)) if fused else int(rng.integers(0, 4))
    qscale = float(rng.uniform(1.0, 10.0))
    proxy = R.PAMA if (not fused and rng.random() < 0.15) else R.CENTROID
    return d, bq, bk, dt, grid, mode, tau, n_text, hil, B, H, fused, mk, mn, qscale, proxy


@pytest.mark.parametrize("seed", range(48), ids=[f"rand_{i:02d}" for i in range(48)])
def test_random_config_parity(seed):
    """Seeded random configurations against the oracle: masks outside the
    rounding band, every output row and LSE, lists against the mask."""
    d, bq, bk, dt, grid, mode, tau, n_text, hil, B, H, fused, mk, mn, qscale, proxy = _random_case(seed)
    w = S.small(f"rand{seed}", B, H, d, grid, bq, bk, tau, dtype=dt, qscale=qscale, n_text=n_text, hilbert=hil,
                cfg_id=200 + seed)
    cfg = cfg_for(w, mode=mode, max_keep=mk, min_keep=mn, fused=fused, proxy=proxy)
    rt, O, L, mask = full_check(w, cfg, label=f"random{' fused' if fused else ''}{' pama' if proxy == R.PAMA else ''}")
    if mn >= 1:
        assert (rt.kv_count.cpu().numpy() >= min(mn, rt.n_kb)).all()


# PAMA proxy (PARK page, section 5.1): per-query block attention averaged in the
# query block; the same selection rules on s = ln A
PAMA_SMALL = [
    # name, grid, d, bq, bk, dtype, tau, mode, max_keep, min_keep, n_text, hilbert, B, H
    ("pama_rel", (4, 8, 32), 128, 128, 128, "bf16", 0.05, R.RELATIVE, 0, 1, 0, False, 1, 2),
    ("pama_topp_cap", (5, 8, 25), 128, 128, 64, "bf16", 0.1, R.TOPP, 6, 1, 0, False, 1, 2),
    ("pama_abs_d64_q64", (3, 9, 21), 64, 64, 128, "bf16", 0.02, R.ABSOLUTE, 0, 2, 0, False, 2, 1),
    ("pama_prefix_hilbert", (4, 8, 30), 128, 128, 128, "bf16", 0.1, R.TOPP, 0, 1, 100, True, 1, 2),
    ("pama_f32", (4, 8, 16), 64, 64, 64, "f32", 0.1, R.TOPP, 0, 1, 0, False, 1, 2),
    ("pama_f32_d128_q128", (3, 7, 19), 128, 128, 64, "f32", 0.02, R.RELATIVE, 3, 1, 0, False, 1, 1),
    ("pama_n130", (1, 10, 13), 128, 128, 64, "bf16", 0.05, R.RELATIVE, 0, 1, 0, False, 1, 1),
    ("pama_n1", (1, 1, 1), 128, 128, 128, "bf16", 0.01, R.TOPP, 0, 1, 0, False, 1, 1),
]


@pytest.mark.parametrize("case", PAMA_SMALL, ids=[c[0] for c in PAMA_SMALL])
def test_pama_parity(case):
    name, grid, d, bq, bk, dt, tau, mode, mk, mn, n_text, hil, B, H = case
    w = S.small(name, B, H, d, grid, bq, bk, tau, dtype=dt, qscale=6.0, n_text=n_text, hilbert=hil)
    cfg = cfg_for(w, mode=mode, max_keep=mk, min_keep=mn, proxy=R.PAMA)
    full_check(w, cfg, label="pama")


# Fused routing (Sol-Attn abstract: selection inside the attention pass, after a
# pre-pass of the proxy row statistics): the same decisions as the two-kernel
# route, taken per work item inside the forward kernel
FUSED_SMALL = [
    # name, grid, d, bq, bk, dtype, tau, mode, min_keep, n_text, hilbert, B, H
    ("fused_rel", (4, 8, 32), 128, 128, 128, "bf16", 0.01, R.RELATIVE, 1, 0, False, 1, 2),
    ("fused_abs_k64", (5, 8, 25), 128, 128, 64, "bf16", 0.01, R.ABSOLUTE, 0, 0, False, 1, 2),
    ("fused_prefix_hilbert", (4, 8, 30), 128, 128, 128, "bf16", 0.01, R.RELATIVE, 1, 100, True, 1, 2),
    ("fused_d64_q64", (3, 9, 21), 64, 64, 128, "bf16", 0.02, R.RELATIVE, 0, 0, False, 2, 1),
    ("fused_f32", (4, 8, 16), 64, 64, 64, "f32", 0.02, R.RELATIVE, 1, 0, False, 1, 2),
    ("fused_all_dropped", (3, 8, 27), 128, 128, 128, "bf16", 2.0, R.RELATIVE, 0, 0, False, 1, 1),
    ("fused_n130", (1, 10, 13), 128, 128, 64, "bf16", 0.05, R.ABSOLUTE, 0, 0, False, 1, 1),
    # a floor of one block: at tau = 1 only the row maximum clears tau, and the
    # fused score of the argmax may round below the pre-pass maximum; with a high
    # ABSOLUTE tau or tau > 1 nothing clears it; the row keeps its best block
    ("fused_rel_tau1_floor", (4, 8, 32), 128, 128, 128, "bf16", 1.0, R.RELATIVE, 1, 0, False, 1, 2),
    ("fused_abs_floor_k64", (5, 8, 25), 128, 128, 64, "bf16", 0.5, R.ABSOLUTE, 1, 0, False, 1, 2),
    ("fused_floor_prefix", (4, 8, 30), 128, 128, 128, "bf16", 2.0, R.RELATIVE, 1, 100, True, 1, 1),
]


@pytest.mark.parametrize("case", FUSED_SMALL, ids=[c[0] for c in FUSED_SMALL])
def test_fused_parity(case):
    name, grid, d, bq, bk, dt, tau, mode, mn, n_text, hil, B, H = case
    w = S.small(name, B, H, d, grid, bq, bk, tau, dtype=dt, qscale=6.0, n_text=n_text, hilbert=hil)
    cfg = cfg_for(w, mode=mode, max_keep=0, min_keep=mn, fused=True)
    rt, O, L, mask = full_check(w, cfg, label="fused")
    if mn >= 1:
        assert (rt.kv_count.cpu().numpy() >= 1).all(), "a row kept no block under a floor of one"
    # the two-kernel route on the same inputs: the same decisions outside the
    # band, and then the same tiles in the same order, so the same bits
    Qc, Kc, Vc, Q, K, V = make(w)
    cfg2 = cfg_for(w, mode=mode, max_keep=0, min_keep=mn)
    rt2, O2, L2 = run_gpu(Q, K, V, cfg2)
    mask2 = rt2.mask().cpu().numpy()
    same = (mask == mask2).all(axis=-1)                  # [B, H, n_qb]: rows with identical decisions
    say(f"  rows with identical decisions {int(same.sum())} / {same.size}")
    rows = torch.from_numpy(np.repeat(same, w.block_q, axis=-1)[..., :w.N])
    assert torch.equal(O.cpu()[rows], O2.cpu()[rows]) and torch.equal(L.cpu()[rows], L2.cpu()[rows])
    # the pre-pass costs each row under the same decisions: equal costs on those
    # rows, and a work order sorted by cost band
    cost, cost2 = rt.cost.cpu().numpy(), rt2.cost.cpu().numpy()
    if not cfg.no_residual:
        assert np.array_equal(cost[same], cost2[same])
    check_work_order(rt)


def test_fused_rejects_what_it_cannot_decide_alone():
    m = sa()
    w = S.small("fr", 1, 1, 128, (2, 8, 16), 128, 128, 0.01)
    Qc, Kc, Vc, Q, K, V = make(w)
    for kw in (dict(max_keep=3), dict(tau_mode=R.TOPP), dict(tau_mode=R.ABSOLUTE, min_keep=2),
               dict(proxy=R.PAMA), dict(tau=1.5, min_keep=2)):
        base = dict(block_q=128, block_k=128, tau=0.01, fused=True, min_keep=0)
        base.update(kw)
        with pytest.raises(m.SparseAttnError) as ei:
            m.route(Q, K, V, m.Config(**base))
        assert ei.value.status == m.binding.SA_ERR_UNSUPPORTED


def test_route_of_other_parameters_refused():
    """A route serves forwards of its own parameters only: a fused route (no lists)
    under a two-kernel forward, or a route of another shape, tau or block size,
    is refused before anything is enqueued; so are out= tensors of another shape."""
    m = sa()
    w = S.small("rp", 1, 2, 128, (2, 8, 16), 128, 128, 0.01)
    Qc, Kc, Vc, Q, K, V = make(w)
    cfg = cfg_for(w)
    fused = cfg_for(w, fused=True)
    rt_f = m.route(Q, K, V, fused)
    with pytest.raises(ValueError, match="other parameters"):
        m.forward(Q, K, V, rt_f, cfg)
    rt = m.route(Q, K, V, cfg)
    for bad in (cfg_for(w, tau=0.02), m.Config(block_q=128, block_k=64, tau=0.01)):
        with pytest.raises(ValueError, match="other parameters"):
            m.forward(Q, K, V, rt, bad)
    with pytest.raises(ValueError):
        m.forward(Q[:, :1].contiguous(), K[:, :1].contiguous(), V[:, :1].contiguous(), rt, cfg)
    with pytest.raises(ValueError, match="out"):
        m.forward(Q, K, V, rt, cfg, out=torch.empty_like(Q[:, :1]))
    with pytest.raises(ValueError, match="other parameters"):
        m.route(Q, K, V, m.Config(block_q=128, block_k=64, tau=0.01), out=rt)
    torch.cuda.synchronize()
    # re-routing into the same buffers with a new tau is allowed, and the route
    # then serves forwards of that tau
    cfg2 = cfg_for(w, tau=0.05)
    m.route(Q, K, V, cfg2, out=rt)
    O = m.forward(Q, K, V, rt, cfg2)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all()


@pytest.mark.parametrize("mode", [R.RELATIVE, R.ABSOLUTE])
def test_tiny_workload(mode):
    w = S.WORKLOADS["tiny"]
    full_check(w, cfg_for(w, mode=mode), label="tiny")


def test_no_residual_flag():
    w = S.small("nr", 1, 2, 128, (4, 8, 32), 128, 64, 0.02)
    full_check(w, cfg_for(w, no_residual=True), label="no-residual")


# ----------------------------------------------------------------------------- early residual test
def _residual_norm_max(rt):
    """Largest Euclidean norms, per residual tile, of its key means as the
    forward forms them (bf16 part plus remainder) and of its remainder rows,
    in fp64 from the route's own tiles: [B, H, words, 2]."""
    t = rt.kv_split[:, :, 0].cpu().double()                 # [B, H, words, 64, d]
    hi, lo = t[:, :, :, :32], t[:, :, :, 32:]
    return torch.stack([(hi + lo).pow(2).sum(-1).sqrt().amax(-1), lo.pow(2).sum(-1).sqrt().amax(-1)], -1)


@pytest.mark.parametrize("d,bq,bk,dt,fused", [(128, 128, 64, "bf16", False), (64, 64, 128, "bf16", False),
                                              (128, 128, 128, "bf16", True), (64, 64, 64, "f32", False)])
def test_residual_bounds(d, bq, bk, dt, fused):
    """k_bounds bounds the norms of every residual tile's key means and of its
    remainder rows from above, within 2^-9 of the largest (zero for tiles past
    the last block)."""
    w = S.small("lob", 2, 3, d, (5, 9, 29), bq, bk, 0.02, dtype=dt)
    say(f"[case] residual bounds d{d} {bq}x{bk} {dt} fused={fused} N{w.N}")
    _, _, _, Q, K, V = make(w)
    rt = sa().route(Q, K, V, cfg_for(w, fused=fused))
    torch.cuda.synchronize()
    ref = _residual_norm_max(rt)
    got = rt.k_bounds.cpu().double()
    assert (got >= ref).all() and (got <= ref * (1 + 2.0 ** -9)).all()


@pytest.mark.parametrize("fused", [False, True])
def test_early_residual_test_changes_nothing(fused):
    """The forward's early tests of a residual tile (from the norms alone, then
    from the key means' bf16 part, with the route's bounds) skip only tiles
    that the full test finds negligible: output and LSE are bitwise those of
    the same forward with the bounds set to +inf, which turns the early tests
    off.  Sharp queries and 64-token key blocks, so that most residual tiles
    are negligible."""
    m = sa()
    w = S.small("skip", 1, 4, 128, (8, 16, 48), 128, 64, 0.02, qscale=12.0)
    say(f"[case] early residual test fused={fused} N{w.N}")
    _, _, _, Q, K, V = make(w)
    cfg = cfg_for(w, fused=fused)
    rt = m.route(Q, K, V, cfg)
    O1, L1 = m.forward(Q, K, V, rt, cfg, lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(rt.k_bounds).all()
    rt.k_bounds.fill_(float("inf"))
    O2, L2 = m.forward(Q, K, V, rt, cfg, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_pama_route_bounds_unused():
    """A PAMA route does not write the remainder bounds and its forward does not
    read them: bounds of NaN (read, they would turn every early test off) and of
    -inf (read, they would skip every residual tile) give bitwise the same
    output and LSE."""
    m = sa()
    w = S.small("pama_lo", 1, 2, 128, (4, 12, 40), 128, 64, 0.1, qscale=4.0)
    say(f"[case] PAMA route ignores the bounds N{w.N}")
    _, _, _, Q, K, V = make(w)
    cfg = cfg_for(w, mode=R.TOPP, proxy=R.PAMA)
    rt = m.route(Q, K, V, cfg)
    rt.k_bounds.fill_(float("nan"))
    O1, L1 = m.forward(Q, K, V, rt, cfg, lse=True)
    rt.k_bounds.fill_(float("-inf"))
    O2, L2 = m.forward(Q, K, V, rt, cfg, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    # control: a centroid route's forward reads them (-inf bounds drop its residual tiles)
    cfg_c = cfg_for(w, mode=R.TOPP)
    rt_c = m.route(Q, K, V, cfg_c)
    O3 = m.forward(Q, K, V, rt_c, cfg_c)
    rt_c.k_bounds.fill_(float("-inf"))
    O4 = m.forward(Q, K, V, rt_c, cfg_c)
    torch.cuda.synchronize()
    assert not torch.equal(O3, O4)


# ----------------------------------------------------------------------------- dense path
@pytest.mark.parametrize("d,bq,bk,dt", [(128, 128, 128, "bf16"), (128, 128, 64, "bf16"), (64, 64, 64, "f32"),
                                        (128, 64, 128, "bf16")])
def test_dense_matches_oracle_and_tau_zero(d, bq, bk, dt):
    m = sa()
    w = S.small("dense", 1, 2, d, (3, 8, 21), bq, bk, 0.0, dtype=dt)
    say(f"[case] dense d{d} {bq}x{bk} {dt} N{w.N}")
    Qc, Kc, Vc, Q, K, V = make(w)
    Od, Ld = m.dense_ref_gpu(Q, K, V, block_q=bq, lse=True)
    cfg = cfg_for(w, tau=0.0)
    rt, O, L = run_gpu(Q, K, V, cfg)
    assert rt.mask().all()
    # tau = 0 keeps every block in ascending order: the same tile sequence as the dense path
    assert torch.equal(O, Od) and torch.equal(L, Ld)
    for h in range(w.H):
        q, k, v = head_np(Qc, 0, h), head_np(Kc, 0, h), head_np(Vc, 0, h)
        O_ref, L_ref = R.dense_ref(q, k, v)
        o = Od[0, h].float().cpu().numpy()
        e_rel = np.linalg.norm(o - O_ref) / np.linalg.norm(O_ref)
        assert e_rel <= 1e-2 and np.abs(o - O_ref).max() <= 3e-2
        assert np.abs(Ld[0, h].cpu().numpy() - L_ref).max() <= 2e-2


# ----------------------------------------------------------------------------- metamorphic
def test_value_shift_and_key_shift():
    """V + 1c^T adds c to every output row (weights sum to one); K + 1c^T shifts each
    row's logits by a constant, leaving mask and output unchanged.  fp32 inputs so
    that the shifted tensors are exact shifts."""
    w = S.small("meta", 1, 2, 128, (4, 8, 32), 128, 64, 0.01, dtype="f32")
    Qc, Kc, Vc, Q, K, V = make(w)
    cfg = cfg_for(w)
    rt, O, _ = run_gpu(Q, K, V, cfg)
    mask0 = rt.mask().cpu().numpy()
    g = torch.Generator().manual_seed(3)
    c = torch.randn(w.d, generator=g)
    rt2, O2, _ = run_gpu(Q, K, (Vc + c).cuda(), cfg)
    assert np.array_equal(rt2.mask().cpu().numpy(), mask0)   # routing never looks at V
    err = (O2.cpu() - O.cpu() - c).abs().max().item()
    assert err <= 1e-2, err
    ck = 0.5 * torch.randn(w.d, generator=g)
    rt3, O3, _ = run_gpu(Q, (Kc + ck).cuda(), V, cfg)
    d3 = rt3.mask().cpu().numpy() != mask0
    for h in range(w.H):
        ort = R.route_ref(head_np(Qc, 0, h), head_np(Kc, 0, h), R.RouteParams(w.block_q, w.block_k, w.tau))
        assert not (d3[0, h] & ~ort.exempt).any()
    if not d3.any():
        e = (O3 - O).abs().max().item()
        assert e <= 1e-2, e


def test_identical_keys_make_residual_exact():
    """Every key of a block equal to its block mean: the residual is exact, so the
    output equals dense attention (keys chosen bf16-representable)."""
    m = sa()
    w = S.small("idk", 1, 2, 128, (4, 8, 30), 128, 64, 0.05)
    Qc, Kc, Vc, _, _, _ = make(w)
    n_kb = -(-w.N // 64)
    reps = torch.repeat_interleave(torch.randn(1, 2, n_kb, 128, generator=torch.Generator().manual_seed(5)), 64, dim=2)
    K2 = (reps[:, :, : w.N] * 2.0).to(torch.bfloat16)
    Q2 = (Qc.float() * 0.5).to(torch.bfloat16)
    cfg = cfg_for(w)
    rt, O, L = run_gpu(Q2.cuda(), K2.cuda(), Vc.cuda(), cfg)
    mask = rt.mask().cpu().numpy()
    assert (~mask).any()
    for h in range(2):
        O_ref, L_ref = R.dense_ref(head_np(Q2, 0, h), head_np(K2, 0, h), head_np(Vc, 0, h))
        o = O[0, h].float().cpu().numpy()
        assert np.linalg.norm(o - O_ref) / np.linalg.norm(O_ref) <= 1e-2
        assert np.abs(o - O_ref).max() <= 3e-2


def _check_means_and_tiles(w, rt, Qc, Kc, Vc):
    """Block means against the oracle's pooling (fp32 accumulation against fp64:
    relative 1e-5) on every head, and the residual tiles: hi rows = bf16 of the
    mean, lo rows = bf16 of the remainder, zero rows past the last block."""
    bq, bk = w.block_q, w.block_k
    qm, km, vm = (t.cpu().double().numpy() for t in (rt.q_mean, rt.k_mean, rt.v_mean))
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = head_np(Qc, b, h), head_np(Kc, b, h), head_np(Vc, b, h)
            for got, ref in ((qm[b, h], R.pool(q, bq)), (km[b, h], R.pool(k, bk)), (vm[b, h], R.pool(v, bk))):
                scale = np.abs(ref).max()
                assert np.abs(got - ref).max() <= 1e-5 * scale, (b, h)
    split = rt.kv_split.cpu()                                  # [B, H, 2, words, 64, d]
    n_kb = rt.n_kb
    for which, means in ((0, rt.k_mean), (1, rt.v_mean)):
        mf = means.cpu()                                       # [B, H, n_kb, d] fp32
        hi = mf.to(torch.bfloat16)
        lo = (mf - hi.float()).to(torch.bfloat16)
        t = split[:, :, which].reshape(w.B, w.H, -1, 64, w.d)  # [B, H, groups, 64, d]
        rows = t.shape[2] * 32
        got_hi = t[:, :, :, :32].reshape(w.B, w.H, rows, w.d)
        got_lo = t[:, :, :, 32:].reshape(w.B, w.H, rows, w.d)
        assert torch.equal(got_hi[:, :, :n_kb], hi) and torch.equal(got_lo[:, :, :n_kb], lo), which
        assert not got_hi[:, :, n_kb:].any() and not got_lo[:, :, n_kb:].any(), which


@pytest.mark.parametrize("dt,bq,bk", [("bf16", 128, 64), ("f32", 64, 128)])
def test_route_means_and_residual_tiles(dt, bq, bk):
    """The route's block means and residual tiles on a small launch (the pool
    kernel pools keys and values, the select kernel the queries)."""
    w = S.small("means", 1, 2, 64 if dt == "f32" else 128, (3, 7, 19), bq, bk, 0.01, dtype=dt)
    say(f"[case] means {dt} {bq}x{bk} N{w.N}")
    Qc, Kc, Vc, Q, K, V = make(w)
    rt, _, _ = run_gpu(Q, K, V, cfg_for(w))
    _check_means_and_tiles(w, rt, Qc, Kc, Vc)


@pytest.mark.parametrize("B,H,grid,bq,bk,dt", [(1, 256, (5, 7, 233), 64, 128, "bf16"),
                                               (2, 256, (1, 13, 315), 64, 64, "f32")])
def test_route_means_large_launch(B, H, grid, bq, bk, dt):
    """The same checks on launches of 2048 select workgroups (16 query blocks
    each, pooled by the workgroup itself) over 256 and 512 heads; ragged last
    blocks (N = 8155 and 4095)."""
    w = S.small("means_big", B, H, 64, grid, bq, bk, 0.01, dtype=dt)
    say(f"[case] means large launch {dt} B{B} H{H} N{w.N} {bq}x{bk}")
    Qc, Kc, Vc, Q, K, V = make(w)
    rt, _, _ = run_gpu(Q, K, V, cfg_for(w))
    _check_means_and_tiles(w, rt, Qc, Kc, Vc)


def test_deterministic_and_route_reuse():
    m = sa()
    w = S.small("det", 1, 3, 128, (4, 8, 32), 128, 64, 0.01, max_keep_frac=0.1)
    _, _, _, Q, K, V = make(w)
    cfg = cfg_for(w)
    rt1, O1, L1 = run_gpu(Q, K, V, cfg)
    rt2, O2, L2 = run_gpu(Q, K, V, cfg)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    for name in ("kv_count", "kv_mask", "row_stats", "q_mean", "k_mean", "v_mean", "cost"):
        assert torch.equal(getattr(rt1, name), getattr(rt2, name)), name
    # a route serves several forward calls, and route buffers can be refilled in place
    O3 = m.forward(Q, K, V, rt1, cfg)
    m.route(Q, K, V, cfg, out=rt2)
    O4 = m.forward(Q, K, V, rt2, cfg)
    torch.cuda.synchronize()
    assert torch.equal(O3, O1) and torch.equal(O4, O1)


def test_side_stream():
    m = sa()
    w = S.small("stream", 1, 2, 128, (4, 8, 32), 128, 128, 0.01)
    _, _, _, Q, K, V = make(w)
    cfg = cfg_for(w)
    rt0, O0, _ = run_gpu(Q, K, V, cfg)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rt = m.route(Q, K, V, cfg)
        O = m.forward(Q, K, V, rt, cfg)
    s.synchronize()
    assert torch.equal(O, O0)


def test_work_order_by_cost_band():
    """Forward schedule written by route: the cost of each query block, and the items
    sorted stably by cost band floor(log2(cost)), highest band first."""
    w = S.small("sched", 1, 4, 128, (4, 8, 32), 128, 64, 0.01)
    say(f"[case] schedule {w.name} H{w.H} N{w.N}")
    _, _, _, Q, K, V = make(w)
    rt, O1, _ = run_gpu(Q, K, V, cfg_for(w))
    wo = rt.work_order.cpu().numpy()
    cost = rt.cost.cpu().numpy().ravel().astype(np.int64)
    # cost = 64-token tiles of kept blocks + one residual tile per 32 pooled blocks
    # holding a dropped block
    mask = rt.mask().cpu().numpy().reshape(-1, rt.n_kb)
    nj = np.minimum(np.arange(rt.n_kb) * 64 + 64, w.N) - np.arange(rt.n_kb) * 64
    tiles = (mask * ((nj + 63) // 64)).sum(axis=1)
    n32 = -(-rt.n_kb // 32)
    pad = np.zeros((mask.shape[0], n32 * 32), dtype=bool)
    pad[:, : rt.n_kb] = ~mask
    tiles += pad.reshape(mask.shape[0], -1, 32).any(axis=2).sum(axis=1)
    assert np.array_equal(cost, tiles)
    band = np.floor(np.log2(np.maximum(cost, 1))).astype(np.int64)
    assert len(np.unique(band)) > 1          # the case exercises more than one band
    assert np.array_equal(wo, np.lexsort((np.arange(cost.size), -band)))
    # the order is a pure function of the costs: a second route gives the same list
    rt2 = sa().route(Q, K, V, cfg_for(w))
    torch.cuda.synchronize()
    assert torch.equal(rt2.work_order, rt.work_order)


def _spread_heads(B, H, N, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    # a random direction per 64-token block, shared by its queries and keys, so
    # that block means are informative; query scales from flat to peaked heads
    E = torch.randn(B, H, N // 64, 1, d, device="cuda", generator=g).expand(B, H, N // 64, 64, d).reshape(B, H, N, d)
    s = torch.linspace(0.05, 1.5, H, device="cuda").view(1, H, 1, 1)
    Q = (s * (E + 0.5 * torch.randn(B, H, N, d, device="cuda", generator=g))).to(torch.bfloat16)
    K = (E + 0.5 * torch.randn(B, H, N, d, device="cuda", generator=g)).to(torch.bfloat16)
    V = torch.randn(B, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
    return Q, K, V


def test_work_order_large():
    """A long work list (30720 items, past the head-major threshold): heads by total
    cost, then cost band, then query block.  Head 1 repeats head 0, so two heads
    tie on total cost (the lower head goes first); per-head query scales spread the
    costs over many bands."""
    m = sa()
    B, H, N, d = 1, 240, 8192, 64
    say(f"[case] schedule large B{B} H{H} N{N} d{d}")
    Q, K, V = _spread_heads(B, H, N, d, 7)
    for T in (Q, K, V):
        T[:, 1] = T[:, 0]
    rt = m.route(Q, K, V, m.Config(block_q=64, block_k=64, tau=0.02))
    torch.cuda.synchronize()
    cost = rt.cost.cpu().numpy()
    assert cost.size == B * H * (N // 64) and cost.size >= 16 * 768
    assert np.array_equal(cost[0, 0], cost[0, 1])
    band = np.floor(np.log2(np.maximum(cost, 1))).astype(np.int64)
    assert len(np.unique(band)) > 3
    check_work_order(rt)
    wo = rt.work_order.cpu().numpy()
    n_qb = cost.shape[-1]
    heads_in_order = wo[::n_qb] // n_qb
    assert np.all(wo.reshape(B * H, n_qb) // n_qb == heads_in_order[:, None])   # each head contiguous
    assert list(heads_in_order).index(0) < list(heads_in_order).index(1)


@pytest.mark.parametrize("BH,N,bq", [(24, 2048 * 64, 64), (1024, 12 * 64, 64)],
                         ids=["items_49152_nqb_2048", "heads_1024_items_12288"])
def test_work_order_head_major_limits(BH, N, bq):
    """The head-major order at its limits: 49152 items with 2048 query blocks per
    head (a whole head's costs in one wave's registers, every thread of the
    placing workgroup holding 48 items), and 1024 heads at the 12288-item
    threshold (a thread per head ranking all heads)."""
    m = sa()
    say(f"[case] schedule limits BH{BH} N{N} block_q{bq}")
    Q, K, V = _spread_heads(1, BH, N, 64, 13)
    rt = m.route(Q, K, V, m.Config(block_q=bq, block_k=64, tau=0.02))
    torch.cuda.synchronize()
    cost = rt.cost.cpu().numpy()
    n_qb = cost.shape[-1]
    assert cost.size in (16 * 768, 48 * 1024) and n_qb <= 32 * 64
    check_work_order(rt)
    wo = rt.work_order.cpu().numpy()
    heads_in_order = wo[::n_qb] // n_qb
    assert np.all(wo.reshape(BH, n_qb) // n_qb == heads_in_order[:, None])   # each head contiguous
    del Q, K, V
    torch.cuda.empty_cache()


def test_work_order_band_tiles():
    """A long work list with more heads than the head-major order takes (1100 >
    1024; also more than its 49152 items): the global cost-band order, with more
    items than the ordering workgroup's 448 tiles of 64 hold (two-chunk tiles,
    chunks loaded in several batches)."""
    m = sa()
    B, H, N, d = 1, 1100, 4096, 64
    say(f"[case] schedule band tiles B{B} H{H} N{N} d{d}")
    Q, K, V = _spread_heads(B, H, N, d, 11)
    rt = m.route(Q, K, V, m.Config(block_q=64, block_k=64, tau=0.02))
    torch.cuda.synchronize()
    cost = rt.cost.cpu().numpy()
    assert cost.size > 64 * 448
    check_work_order(rt)


def test_work_order_many_items():
    """More items than the ordering workgroup has threads, with ragged chunks."""
    w = S.small("sched_many", 2, 6, 64, (5, 12, 45), 64, 64, 0.02)
    say(f"[case] schedule {w.name} B{w.B} H{w.H} N{w.N}")
    _, _, _, Q, K, V = make(w)
    rt, _, _ = run_gpu(Q, K, V, cfg_for(w))
    cost = rt.cost.cpu().numpy().ravel().astype(np.int64)
    assert cost.size > 512 and cost.size % 512
    check_work_order(rt)
