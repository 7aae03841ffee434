"""CPU oracle for block-sparse attention with routing and a dropped-block residual.

TEST INFRASTRUCTURE, not product code.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything here.  It is independent of
the HIP library and its binding: no shared kernels, headers, helpers or
constants.

Modules
  sparse_attn_ref  vectorised float64 numpy oracle (routing, sparse + residual
                   forward, dense attention, attention recall diagnostic)
  brute            scalar loops with exactly rounded sums, for tiny inputs; pins
                   the vectorised oracle

Parity status of each function is recorded beside its pins in tests/; every
function here is pinned by closed forms, library routines, invariants or the
brute-force implementation.
"""
from .sparse_attn_ref import (ABSOLUTE, EXEMPT_BAND, RELATIVE, RouteParams, RouteResult,  # noqa: F401
                              attention_recall, block_counts, dense_ref, forward_ref,
                              forward_ref_with_mask, n_blocks, pool, route_ref)
