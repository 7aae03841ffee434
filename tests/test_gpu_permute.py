"""GPU parity of the token permutation (sparse_attn_permute_tokens) against the
oracle's definition: bit-exact rows, gather and scatter, with a text prefix,
ragged lengths, both dtypes and both head sizes; and the Hilbert round trip of
a routed forward."""
import numpy as np
import pytest
import torch

from oracle import reorder as RO
from tests._gpu_common import say

pytestmark = pytest.mark.gpu


def sa():
    import free_block_sparse_route_amd as m
    return m


CASES = [
    # B, H, N, d, dtype, n0, grid (n_perm = prod(grid)); rows past n0 + n_perm copied
    (1, 2, 64, 64, torch.float32, 0, (2, 4, 8)),
    (2, 3, 37 + 105, 128, torch.bfloat16, 37, (3, 5, 7)),
    (1, 1, 961, 128, torch.bfloat16, 1, (4, 8, 30)),
    (1, 2, 300, 64, torch.float32, 250, (2, 3, 7)),
]


@pytest.mark.parametrize("B,H,N,d,dt,n0,grid", CASES)
@pytest.mark.parametrize("inverse", [False, True])
def test_permute_matches_definition(B, H, N, d, dt, n0, grid, inverse):
    m = sa()
    n = int(np.prod(grid))
    assert n0 + n <= N
    say(f"[case] permute B{B} H{H} N{N} d{d} {dt} n0={n0} grid={grid} inverse={inverse}")
    g = torch.Generator().manual_seed(N + d)
    x = torch.randn(B, H, N, d, generator=g).to(dt)
    perm = m.hilbert_order(*grid)
    want = RO.permute_rows(x.float().numpy(), perm.numpy(), n0, inverse)
    got = m.permute_tokens(x.cuda(), perm.cuda(), n0, inverse)
    torch.cuda.synchronize()
    assert np.array_equal(got.float().cpu().numpy(), want)


def test_permute_round_trip_and_copy_only():
    m = sa()
    x = torch.randn(2, 2, 500, 128).to(torch.bfloat16).cuda()
    perm = torch.randperm(480, generator=torch.Generator().manual_seed(1)).to(torch.int32).cuda()
    y = m.permute_tokens(x, perm, 20)
    z = m.permute_tokens(y, perm, 20, inverse=True)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    c = m.permute_tokens(x, empty, 500)                      # no permuted rows: a copy
    torch.cuda.synchronize()
    assert torch.equal(z, x) and torch.equal(c, x)
    assert not torch.equal(y, x)


def test_permute_skips_entries_outside_the_range():
    m = sa()
    x = torch.randn(1, 1, 8, 64).cuda()
    perm = torch.tensor([1, 0, -1, 99, 4, 5, 6, 7], dtype=torch.int32).cuda()
    out = torch.full_like(x, 7.0)
    m.permute_tokens(x, perm, 0, out=out)
    torch.cuda.synchronize()
    want = x.cpu().clone()
    want[0, 0, 0], want[0, 0, 1] = x[0, 0, 1].cpu(), x[0, 0, 0].cpu()
    want[0, 0, 2:4] = 7.0
    assert torch.equal(out.cpu(), want)


def test_hilbert_round_trip_of_a_routed_forward():
    """Reorder the video tokens of raster-order inputs, route and attend, restore
    the order: equal to running the same pipeline on inputs the generator put
    in Hilbert order and un-permuting on the host."""
    m = sa()
    from workloads import synth as S
    w = S.small("hil", 1, 2, 128, (4, 8, 16), 128, 128, 0.02, n_text=64, hilbert=True)
    wr = w.with_(hilbert=False)
    Qh, Kh, Vh = (t.cuda() for t in S.make_qkv(w))           # generator's Hilbert order
    Qr, Kr, Vr = (t.cuda() for t in S.make_qkv(wr))          # raster order
    perm = m.hilbert_order(*w.grid).cuda()
    n0 = w.n_text
    say("[case] hilbert round trip", w.grid, "n0", n0)
    q2, k2, v2 = (m.permute_tokens(t, perm, n0) for t in (Qr, Kr, Vr))
    assert torch.equal(q2, Qh) and torch.equal(k2, Kh) and torch.equal(v2, Vh)
    cfg = m.Config(block_q=128, block_k=128, tau=w.tau, n_dense_prefix=n0)
    o_h = m.forward(q2, k2, v2, m.route(q2, k2, v2, cfg), cfg)
    o = m.permute_tokens(o_h, perm, n0, inverse=True)
    torch.cuda.synchronize()
    want = RO.permute_rows(o_h.float().cpu().numpy(), perm.cpu().numpy(), n0, inverse=True)
    assert np.array_equal(o.float().cpu().numpy(), want)
