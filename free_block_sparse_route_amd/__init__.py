"""Block-sparse attention with block routing and a dropped-block residual,
hand-written HIP for AMD Instinct MI355X (gfx950).

    import free_block_sparse_route_amd as sa
    cfg = sa.Config(block_q=128, block_k=128, tau=0.01)
    rt = sa.route(q, k, v, cfg)          # block means, proxy rows, keep lists
    o = sa.forward(q, k, v, rt, cfg)     # kept tiles exactly, dropped blocks by residual
    o_dense = sa.dense_ref_gpu(q, k, v)  # same kernels, every block kept, no residual

q, k, v: device tensors [B, H, N, d], bf16 or fp32, d in {64, 128}.

Hilbert token order (video grid T x Hh x W after an n0-token prefix):
    perm = sa.hilbert_order(T, Hh, W).cuda()
    qh = sa.permute_tokens(q, perm, n0)                 # and k, v
    o = sa.permute_tokens(o_h, perm, n0, inverse=True)  # back to raster order
"""
from .binding import (ABSOLUTE, CENTROID, FLAG_FUSED, FLAG_NO_RESIDUAL, FLAG_PAMA, PAMA, RELATIVE, TOPP, Config, Route, SaParams, SaRoute,  # noqa: F401
                      SparseAttnError, dense_flops, dense_ref_gpu, forward, forward_sparsepr, forward_sparsepr_static,
                      hilbert_order,
                      kv_idx_cap, last_error, make_params, permute_tokens, route, route_sizes,
                      sparsepr_workspace_size, status_string)
