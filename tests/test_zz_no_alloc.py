"""The allocation-free probe-fitted entry point (sparse_attn_forward_sparsepr_static)
against the workspace entry point (sparse_attn_forward_sparsepr) through the C ABI:
two calls in a row, the second on a smaller input, each within the output
tolerance of the workspace call on the same route (and against the oracle on
one head).  Sizes beyond the static array are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import sparsepr as SP
from workloads import synth as S

from _gpu_common import MAX_ABS, REL_FRO, cfg_for, head_np, oracle_params, rel_fro, sa, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _pair(m, w, P, rank, ridge, check_oracle):
    say(f"[case] no-alloc sparsepr {w.name} B{w.B} H{w.H} N{w.N} d{w.d} {w.block_q}x{w.block_k} P={P}")
    Qc, Kc, Vc = S.make_qkv(w)
    Q, K, V = Qc.cuda(), Kc.cuda(), Vc.cuda()
    cfg = cfg_for(w)
    rt = m.route(Q, K, V, cfg)
    O_ws = m.forward_sparsepr(Q, K, V, rt, cfg, probes_per_block=P, rank=rank, ridge=ridge)
    O_st = m.forward_sparsepr_static(Q, K, V, rt, cfg, probes_per_block=P, rank=rank, ridge=ridge)
    torch.cuda.synchronize()
    a, b = O_st.float().cpu().numpy(), O_ws.float().cpu().numpy()
    assert np.isfinite(a).all()
    e_rel, e_abs = rel_fro(a, b), float(np.abs(a - b).max())
    say(f"   static vs workspace: rel-fro {e_rel:.2e}, max-abs {e_abs:.2e}, bitwise {np.array_equal(a, b)}")
    assert e_rel <= REL_FRO and e_abs <= MAX_ABS
    if check_oracle:
        mask = rt.mask().cpu().numpy()
        want, _ = SP.sparsepr_ref(head_np(Qc, 0, 0), head_np(Kc, 0, 0), head_np(Vc, 0, 0), mask[0, 0],
                                  oracle_params(cfg), P, rank, ridge)
        # end to end against the oracle's own intermediates: relative Frobenius (the
        # fit's conditioning makes max-abs there a property of the inputs' rounding)
        e = rel_fro(a[0, 0], want)
        assert e <= REL_FRO, e


def test_static_matches_workspace_twice_then_smaller():
    m = sa()
    big = S.small("na_big", 1, 3, 128, (6, 10, 160), 128, 128, 0.01)      # N = 9600, 300 probes a head
    small = S.small("na_small", 1, 1, 64, (3, 8, 20), 64, 64, 0.05)      # N = 480
    _pair(m, big, 4, 8, 1e-3, True)
    _pair(m, small, 2, 4, 1e-2, True)


def test_static_refuses_what_does_not_fit():
    """A call whose workspace exceeds the static array, even with one key range
    for the probe pass, is SA_ERR_CAPACITY before anything is enqueued."""
    m = sa()
    B = m.binding
    # 64 heads of N = 32760, d = 128: the sparse pass's fp32 output alone is 1 GiB
    p = B.SaParams(1, 64, 32760, 128, 128, 128, 0.01, 0, 0, 1, 0, 0.0, 0, 0)
    A = 0x1000                     # stand-in device addresses, never dereferenced
    r = B.SaRoute(*([A] * len(B.BUFFERS)), 256)
    st = B.lib.sparse_attn_forward_sparsepr_static(ctypes.byref(p), A, A, A, ctypes.byref(r), 4, 8, 1e-3, A, None)
    assert st == B.SA_ERR_CAPACITY and "static" in B.last_error()
