"""GPU parity of the probe-fitted residual correction (sparse_attn_forward_sparsepr)
against the oracle (oracle/sparsepr.py) on the GPU route's own masks, and its
error next to the proxy-reuse residual's, both against dense attention."""
import numpy as np
import pytest
import torch

from oracle import sparse_attn_ref as R
from oracle import sparsepr as SP
from workloads import synth as S

from _gpu_common import MAX_ABS, REL_FRO, cfg_for, head_np, oracle_params, rel_fro, sa, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    # name, grid, d, bq, bk, dtype, query scale, tau, probes per block, rank, ridge, B, H
    ("pr_r128", (4, 8, 32), 128, 128, 128, "bf16", 6.0, 0.02, 2, 8, 1e-3, 1, 2),
    ("pr_k64_ragged", (5, 8, 25), 128, 128, 64, "bf16", 6.0, 0.01, 4, 4, 1e-2, 1, 2),
    ("pr_d64_q64", (3, 9, 21), 64, 64, 128, "bf16", 6.0, 0.05, 3, 16, 1e-3, 2, 1),
    ("pr_f32", (4, 8, 16), 64, 64, 64, "f32", 6.0, 0.05, 2, 8, 1e-3, 1, 1),
    ("pr_rank1_many_probes", (2, 8, 20), 128, 128, 64, "bf16", 6.0, 0.05, 16, 1, 1e-1, 1, 1),
    # flatter attention (query scale 1.5) and a high tau: the dropped blocks carry real
    # mass, so the corrections differ from one another and from no correction
    ("pr_flat", (4, 8, 32), 128, 128, 64, "bf16", 1.5, 0.3, 4, 8, 1e-3, 1, 2),
    ("pr_flat_f32", (4, 8, 16), 64, 64, 64, "f32", 1.5, 0.3, 4, 8, 1e-3, 1, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sparsepr_parity(case):
    name, grid, d, bq, bk, dt, qs, tau, P, rank, ridge, B, H = case
    m = sa()
    w = S.small(name, B, H, d, grid, bq, bk, tau, dtype=dt, qscale=qs)
    say(f"[case] sparsepr {name} N{w.N} d{d} {bq}x{bk} {dt} tau={tau} P={P} rank={rank} ridge={ridge}")
    Qc, Kc, Vc = S.make_qkv(w)
    Q, K, V = Qc.cuda(), Kc.cuda(), Vc.cuda()
    cfg = cfg_for(w)
    rt = m.route(Q, K, V, cfg)
    O = m.forward_sparsepr(Q, K, V, rt, cfg, probes_per_block=P, rank=rank, ridge=ridge)
    Oblk = m.forward(Q, K, V, rt, cfg)
    torch.cuda.synchronize()
    mask = rt.mask().cpu().numpy()
    Oc, Ob = O.float().cpu().numpy(), Oblk.float().cpu().numpy()
    assert np.isfinite(Oc).all()
    p = oracle_params(cfg)
    for b in range(B):
        for h in range(H):
            q, k, v = head_np(Qc, b, h), head_np(Kc, b, h), head_np(Vc, b, h)
            want, (Os, probes, Od, *_) = SP.sparsepr_ref(q, k, v, mask[b, h], p, P, rank, ridge)
            e_rel, e_abs = rel_fro(Oc[b, h], want), float(np.abs(Oc[b, h] - want).max())
            assert e_rel <= REL_FRO and e_abs <= MAX_ABS, f"rel-Frobenius {e_rel:.3e}, max-abs {e_abs:.3e}"
            dense, _ = R.dense_ref(q, k, v)
            np.testing.assert_allclose(Oc[b, h][probes], dense[probes], atol=MAX_ABS)
            say(f"   b{b} h{h}: GPU vs oracle rel-fro {e_rel:.2e}; against dense attention: oracle kept "
                f"tokens only {rel_fro(Os, dense):.2e}, oracle probe-fitted {rel_fro(want, dense):.2e}, GPU "
                f"probe-fitted {rel_fro(Oc[b, h], dense):.2e}, GPU block residual {rel_fro(Ob[b, h], dense):.2e}")


def test_sparsepr_everything_kept_is_dense():
    """tau = 0 keeps every block: nothing to correct, the output is dense attention."""
    m = sa()
    w = S.small("pr_dense", 1, 1, 128, (2, 8, 16), 128, 128, 0.0, qscale=6.0)
    Qc, Kc, Vc = S.make_qkv(w)
    Q, K, V = Qc.cuda(), Kc.cuda(), Vc.cuda()
    cfg = cfg_for(w, tau=0.0)
    O = m.forward_sparsepr(Q, K, V, m.route(Q, K, V, cfg), cfg, probes_per_block=2, rank=4)
    D = m.dense_ref_gpu(Q, K, V)
    torch.cuda.synchronize()
    dense, _ = R.dense_ref(head_np(Qc, 0, 0), head_np(Kc, 0, 0), head_np(Vc, 0, 0))
    assert rel_fro(O[0, 0].float().cpu().numpy(), dense) <= REL_FRO
    assert torch.allclose(O.float(), D.float(), atol=2e-2)
