"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, agrees with a C compiler on struct layout, and rejects bad
arguments on the host before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

sa = pytest.importorskip("free_block_sparse_route_amd")
B = sa.binding


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 12, names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "sparse_attn.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %d\\n\", sizeof(sa_params), sizeof(sa_route),"
        " offsetof(sa_params, flags), offsetof(sa_route, kv_idx_cap), offsetof(sa_route, work_order),"
        " offsetof(sa_params, scale), SA_ROUTE_NBUF);return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    vals = [int(x) for x in out]
    assert vals[0] == ctypes.sizeof(B.SaParams)
    assert vals[1] == ctypes.sizeof(B.SaRoute)
    assert vals[2] == B.SaParams.flags.offset
    assert vals[3] == B.SaRoute.kv_idx_cap.offset
    assert vals[4] == B.SaRoute.work_order.offset
    assert vals[5] == B.SaParams.scale.offset
    assert vals[6] == len(B.BUFFERS)


def params(**kw):
    base = dict(B=1, H=2, N=1000, d=128, block_q=128, block_k=64, tau=0.01, tau_mode=0, max_keep=0, min_keep=1,
                n_dense_prefix=0, scale=0.0, dtype=0, flags=0)
    base.update(kw)
    return B.SaParams(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), B.SA_ERR_INVALID_ARG), (dict(B=0), B.SA_ERR_INVALID_ARG), (dict(tau=-1.0), B.SA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), B.SA_ERR_INVALID_ARG), (dict(tau_mode=3), B.SA_ERR_INVALID_ARG), (dict(tau_mode=-1), B.SA_ERR_INVALID_ARG),
    (dict(max_keep=-1), B.SA_ERR_INVALID_ARG), (dict(n_dense_prefix=1001), B.SA_ERR_INVALID_ARG),
    (dict(dtype=5), B.SA_ERR_INVALID_ARG), (dict(flags=8), B.SA_ERR_INVALID_ARG),
    (dict(scale=-1.0), B.SA_ERR_INVALID_ARG), (dict(d=96), B.SA_ERR_UNSUPPORTED),
    (dict(block_q=32), B.SA_ERR_UNSUPPORTED), (dict(block_k=256), B.SA_ERR_UNSUPPORTED),
    (dict(N=2_000_000, block_k=64), B.SA_ERR_UNSUPPORTED),
    # fused routing decides each block alone: no cap, no top-p, no PAMA, no floor above one block
    (dict(flags=4, max_keep=3), B.SA_ERR_UNSUPPORTED), (dict(flags=4, tau_mode=2), B.SA_ERR_UNSUPPORTED),
    (dict(flags=6), B.SA_ERR_UNSUPPORTED), (dict(flags=4, min_keep=2), B.SA_ERR_UNSUPPORTED),
    (dict(flags=4, tau_mode=1, min_keep=3), B.SA_ERR_UNSUPPORTED),
    # one head's keys beyond the 32-bit byte range of the kernels' buffer resources
    (dict(N=8_388_608, d=128, dtype=1, block_k=128), B.SA_ERR_UNSUPPORTED),
])
def test_invalid_params_rejected(kw, status):
    p = params(**kw)
    assert B.lib.sparse_attn_kv_idx_cap(ctypes.byref(p)) == status
    arr = (ctypes.c_size_t * len(B.BUFFERS))()
    assert B.lib.sparse_attn_route_sizes(ctypes.byref(p), 1 << 20, arr) == status
    assert B.lib.sparse_attn_last_error().decode() != ""


def test_fused_floor_configurations_accepted():
    """Fused routing takes a floor of at most one block (the row's best block when
    nothing clears tau), in either tau mode and at any tau."""
    for kw in (dict(flags=4), dict(flags=4, tau_mode=1, min_keep=0), dict(flags=4, tau=1.0),
               dict(flags=5, min_keep=0, tau=3.0), dict(flags=4, tau_mode=1, min_keep=1),
               dict(flags=4, tau=1.5)):
        assert B.lib.sparse_attn_kv_idx_cap(ctypes.byref(params(**kw))) > 0, kw


def test_head_byte_range_limit():
    """The largest head the kernels address (N * d * element size <= 2^32 - 1 bytes)
    is accepted; one token more is rejected before any launch, for the dense path too."""
    A = 0x1000                     # a stand-in device address (16-byte aligned), never dereferenced
    n_ok = (2 ** 32 - 1) // (128 * 4)
    ok = params(N=n_ok, d=128, dtype=1, block_q=128, block_k=128, tau=0.0)
    over = params(N=n_ok + 1, d=128, dtype=1, block_q=128, block_k=128, tau=0.0)
    st = B.lib.sparse_attn_dense_ref_gpu(ctypes.byref(over), A, A, A, A, None, None)
    assert st == B.SA_ERR_UNSUPPORTED and "bytes per head" in B.last_error()
    # the accepted size stops at a later check (no pointers), not at the byte range
    st = B.lib.sparse_attn_dense_ref_gpu(ctypes.byref(ok), A, A, A, None, None, None)
    assert st == B.SA_ERR_INVALID_ARG and "o is NULL" in B.last_error()


def test_route_parameters_checked_by_the_binding():
    """A route remembers the parameters it was built for; a forward with other
    shapes, routing fields or routing flags is refused before anything is
    enqueued (only the forward-only no-residual switch may differ)."""
    p = params(B=1, H=2, N=1000, d=64, block_q=64, block_k=64, flags=B.FLAG_FUSED)
    rt = B.Route(p, "cpu")
    rt.check(p, "forward")
    rt.check(B.SaParams.from_buffer_copy(params(B=1, H=2, N=1000, d=64, block_q=64, block_k=64,
                                                flags=B.FLAG_FUSED | B.FLAG_NO_RESIDUAL)), "forward")
    for kw in (dict(flags=0), dict(N=999), dict(block_k=128), dict(tau=0.02), dict(dtype=1), dict(H=3),
               dict(flags=B.FLAG_FUSED | B.FLAG_PAMA)):
        base = dict(B=1, H=2, N=1000, d=64, block_q=64, block_k=64, flags=B.FLAG_FUSED)
        base.update(kw)
        with pytest.raises(ValueError, match="other parameters"):
            rt.check(params(**base), "forward")


@pytest.mark.parametrize("block_q,dtype,n_max", [(64, 0, 3248), (128, 0, 4330), (64, 1, 4352), (128, 1, 5222)])
def test_pama_key_block_limit(block_q, dtype, n_max):
    """The PAMA workgroup keeps per-wave partial rows, the group's ln A rows and
    the queries' normalisers beside a 26 KB staging tile in at most 128 KB of
    LDS: the largest n_kb is accepted, one more is rejected before any launch."""
    ok = params(flags=2, block_q=block_q, block_k=64, dtype=dtype, N=n_max * 64)
    assert B.lib.sparse_attn_kv_idx_cap(ctypes.byref(ok)) > 0, B.lib.sparse_attn_last_error().decode()
    over = params(flags=2, block_q=block_q, block_k=64, dtype=dtype, N=(n_max + 1) * 64)
    assert B.lib.sparse_attn_kv_idx_cap(ctypes.byref(over)) == B.SA_ERR_UNSUPPORTED
    assert "PAMA" in B.lib.sparse_attn_last_error().decode()


@pytest.mark.parametrize("per,rank,ridge,flags,status", [
    (0, 4, 1e-3, 0, B.SA_ERR_INVALID_ARG), (17, 4, 1e-3, 0, B.SA_ERR_INVALID_ARG),
    (2, 0, 1e-3, 0, B.SA_ERR_INVALID_ARG), (2, 17, 1e-3, 0, B.SA_ERR_INVALID_ARG),
    (2, 4, -1.0, 0, B.SA_ERR_INVALID_ARG), (2, 4, float("inf"), 0, B.SA_ERR_INVALID_ARG),
    (2, 4, 1e-3, 4, B.SA_ERR_UNSUPPORTED),
])
def test_sparsepr_rejects_bad_arguments_before_launch(per, rank, ridge, flags, status):
    p = params(flags=flags)
    r = B.SaRoute(*([0x1000] * len(B.BUFFERS)), 1 << 10)
    st = B.lib.sparse_attn_forward_sparsepr(ctypes.byref(p), 0x1000, 0x1000, 0x1000, ctypes.byref(r), per, rank,
                                            ridge, 0x1000, 1 << 40, 0x1000, None)
    assert st == status, B.lib.sparse_attn_last_error().decode()


def test_sparsepr_workspace_size_and_capacity():
    p = params()
    n = ctypes.c_size_t()
    assert B.lib.sparse_attn_sparsepr_workspace_size(ctypes.byref(p), 2, ctypes.byref(n)) == B.SA_OK
    # N = 1000, d = 128, bf16, B*H = 2, block_q = 128: M = 8 * 2 = 16 probes
    up = lambda x: (x + 255) // 256 * 256
    # gathered queries, dense probe outputs, sparse outputs, Gram matrices, one
    # chunk of Gram matrices and means (16 probes <= 128 per chunk), B, b, and
    # the probe pass in 2 key ranges (2 query blocks; 16 key tiles, >= 8 a range)
    want = (up(2 * 16 * 128 * 2) + up(2 * 16 * 128 * 4) + up(2 * 1000 * 128 * 4) + up(2 * 3 * 128 * 128 * 4)
            + up(2 * 1 * 3 * 128 * 128 * 4) + up(2 * 1 * 2 * 128 * 4) + up(2 * 128 * 128 * 4) + up(2 * 128 * 4)
            + up(2 * 2 * 16 * 128 * 4) + up(2 * 2 * 16 * 4))
    assert n.value == want
    r = B.SaRoute(*([0x1000] * len(B.BUFFERS)), 1 << 10)
    st = B.lib.sparse_attn_forward_sparsepr(ctypes.byref(p), 0x1000, 0x1000, 0x1000, ctypes.byref(r), 2, 4, 1e-3,
                                            0x1000, want - 1, 0x1000, None)
    assert st == B.SA_ERR_CAPACITY


def test_kv_idx_cap_rules():
    assert B.kv_idx_cap(params()) == 16                               # no cap: n_kb = ceil(1000/64)
    assert B.kv_idx_cap(params(max_keep=4)) == 4
    assert B.kv_idx_cap(params(max_keep=4, min_keep=9)) == 9
    assert B.kv_idx_cap(params(max_keep=40)) == 16
    assert B.kv_idx_cap(params(max_keep=4, n_dense_prefix=10)) == 16  # prefix row keeps everything


def test_route_sizes_wan13b():
    p = params(B=1, H=12, N=32760, d=128, block_q=128, block_k=128)
    cap = B.kv_idx_cap(p)
    s = dict(zip(B.BUFFERS, B.route_sizes(p, cap)))
    assert cap == 256
    assert s["kv_count"] == 12 * 256 * 4
    assert s["kv_idx"] == 12 * 256 * 256 * 4
    assert s["kv_mask"] == 12 * 256 * 8 * 4
    assert s["k_mean"] == 12 * 256 * 128 * 4
    assert s["work_order"] == 12 * 256 * 4
    assert s["k_bounds"] == 12 * 8 * 2 * 4
    with pytest.raises(B.SparseAttnError) as e:
        B.route_sizes(p, cap - 1)
    assert e.value.status == B.SA_ERR_CAPACITY


def test_null_pointers_rejected_before_launch():
    p = params()
    r = B.SaRoute()
    A = 0x1000                     # a stand-in device address (16-byte aligned), never dereferenced
    st = B.lib.sparse_attn_route(ctypes.byref(p), None, A, A, ctypes.byref(r), None)
    assert st == B.SA_ERR_INVALID_ARG and "q is NULL" in B.last_error()
    st = B.lib.sparse_attn_route(ctypes.byref(p), A, A, A, ctypes.byref(r), None)
    assert st == B.SA_ERR_INVALID_ARG and "route.kv_count" in B.last_error()
    st = B.lib.sparse_attn_forward(ctypes.byref(p), A, A, A, None, A, None, None)
    assert st == B.SA_ERR_INVALID_ARG and "route is NULL" in B.last_error()
    st = B.lib.sparse_attn_dense_ref_gpu(ctypes.byref(p), A, A, A, None, None, None)
    assert st == B.SA_ERR_INVALID_ARG and "o is NULL" in B.last_error()
    st = B.lib.sparse_attn_route(None, A, A, A, ctypes.byref(r), None)
    assert st == B.SA_ERR_INVALID_ARG


def test_capacity_checked_before_launch():
    p = params(max_keep=4)
    A = 0x1000                     # a stand-in device address (16-byte aligned), never dereferenced
    r = B.SaRoute(*([A] * len(B.BUFFERS)), 3)
    assert B.lib.sparse_attn_route(ctypes.byref(p), A, A, A, ctypes.byref(r), None) == B.SA_ERR_CAPACITY
    assert B.lib.sparse_attn_forward(ctypes.byref(p), A, A, A, ctypes.byref(r), A, None, None) == B.SA_ERR_CAPACITY


def test_status_strings():
    assert B.status_string(0) == "ok"
    assert "capacity" in B.status_string(B.SA_ERR_CAPACITY)
    assert B.status_string(-99) == "unknown status"


def test_misaligned_device_pointers_rejected_before_launch():
    """Device pointers must be 16-byte aligned (the kernels move 16-byte vectors);
    a misaligned one is an argument error, and nothing is launched."""
    p = params()
    good, bad = 0x1000, 0x1008
    r = B.SaRoute(*([good] * len(B.BUFFERS)), 1 << 10)
    assert B.lib.sparse_attn_forward(ctypes.byref(p), bad, good, good, ctypes.byref(r), good, None, None) == \
        B.SA_ERR_INVALID_ARG
    assert b"aligned" in B.lib.sparse_attn_last_error()
    r_bad = B.SaRoute(*([good] * (len(B.BUFFERS) - 1) + [bad]), 1 << 10)      # k_bounds misaligned
    assert B.lib.sparse_attn_route(ctypes.byref(p), good, good, good, ctypes.byref(r_bad), None) == \
        B.SA_ERR_INVALID_ARG
    assert b"k_bounds" in B.lib.sparse_attn_last_error()
    # the forward reads the bounds only of a centroid route with the residual fold
    assert B.lib.sparse_attn_forward(ctypes.byref(p), good, good, good, ctypes.byref(r_bad), good, None, None) == \
        B.SA_ERR_INVALID_ARG
    # a centroid route writes the bounds, also under SA_FLAG_NO_RESIDUAL
    r_null = B.SaRoute(*([good] * (len(B.BUFFERS) - 1) + [0]), 1 << 10)      # k_bounds NULL
    assert B.lib.sparse_attn_route(ctypes.byref(params(flags=B.FLAG_NO_RESIDUAL)), good, good, good,
                                   ctypes.byref(r_null), None) == B.SA_ERR_INVALID_ARG
    assert b"k_bounds" in B.lib.sparse_attn_last_error()
    assert B.lib.sparse_attn_permute_tokens(1, 1, 64, 64, 0, 0, 0, None, 0, bad, good, None) == B.SA_ERR_INVALID_ARG
