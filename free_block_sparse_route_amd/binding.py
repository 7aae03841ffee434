"""ctypes binding of libsparse_attn.so (argument marshalling only).

Same names as the C ABI in include/sparse_attn.h: route, forward,
dense_ref_gpu, route_sizes, kv_idx_cap, hilbert_order, permute_tokens,
forward_sparsepr, sparsepr_workspace_size.  Torch tensors supply device memory
and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  If the library has not been built the import fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_CAPACITY, SA_ERR_HIP = 0, -1, -2, -3, -4
SA_BF16, SA_F32 = 0, 1
RELATIVE, ABSOLUTE, TOPP = 0, 1, 2
FLAG_NO_RESIDUAL = 1
FLAG_PAMA = 2
FLAG_FUSED = 4
CENTROID, PAMA = 0, 1          # routing proxy
BUFFERS = ("kv_count", "kv_idx", "kv_mask", "q_mean", "k_mean", "v_mean", "kv_split", "row_stats", "cost",
           "work_order", "k_bounds")


class SaParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("tau", ctypes.c_float),
                ("tau_mode", ctypes.c_int32), ("max_keep", ctypes.c_int32), ("min_keep", ctypes.c_int32),
                ("n_dense_prefix", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class SaRoute(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BUFFERS] + [("kv_idx_cap", ctypes.c_int32)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} [status {status}]")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python free_block_sparse_route_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, R = ctypes.POINTER(SaParams), ctypes.POINTER(SaRoute)
    vp = ctypes.c_void_p
    lib.sparse_attn_kv_idx_cap.argtypes = [P]
    lib.sparse_attn_kv_idx_cap.restype = ctypes.c_int32
    lib.sparse_attn_route_sizes.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_attn_route_sizes.restype = ctypes.c_int
    lib.sparse_attn_route.argtypes = [P, vp, vp, vp, R, vp]
    lib.sparse_attn_route.restype = ctypes.c_int
    lib.sparse_attn_forward.argtypes = [P, vp, vp, vp, R, vp, vp, vp]
    lib.sparse_attn_forward.restype = ctypes.c_int
    lib.sparse_attn_dense_ref_gpu.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sparse_attn_dense_ref_gpu.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.sparse_attn_hilbert_order.argtypes = [i32, i32, i32, ctypes.POINTER(i32)]
    lib.sparse_attn_hilbert_order.restype = ctypes.c_int
    lib.sparse_attn_permute_tokens.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.sparse_attn_permute_tokens.restype = ctypes.c_int
    lib.sparse_attn_sparsepr_workspace_size.argtypes = [P, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_attn_sparsepr_workspace_size.restype = ctypes.c_int
    lib.sparse_attn_forward_sparsepr.argtypes = [P, vp, vp, vp, R, i32, i32, ctypes.c_float, vp, ctypes.c_size_t,
                                                 vp, vp]
    lib.sparse_attn_forward_sparsepr.restype = ctypes.c_int
    lib.sparse_attn_forward_sparsepr_static.argtypes = [P, vp, vp, vp, R, i32, i32, ctypes.c_float, vp, vp]
    lib.sparse_attn_forward_sparsepr_static.restype = ctypes.c_int
    lib.sparse_attn_status_string.argtypes = [ctypes.c_int]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status: int):
    if status != SA_OK:
        raise SparseAttnError(status, lib.sparse_attn_last_error().decode())


@dataclass
class Config:
    """Routing and attention parameters (the sa_params fields other than shapes)."""
    block_q: int = 128
    block_k: int = 128
    tau: float = 0.0
    tau_mode: int = RELATIVE
    max_keep: int = 0
    min_keep: int = 1
    n_dense_prefix: int = 0
    scale: float = 0.0
    no_residual: bool = False
    proxy: int = CENTROID      # CENTROID (block means) or PAMA (per-query, averaged)
    fused: bool = False        # routing decisions taken inside the forward pass


def make_params(q: torch.Tensor, cfg: Config) -> SaParams:
    B, H, N, d = q.shape
    dt = {torch.bfloat16: SA_BF16, torch.float32: SA_F32}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype} (bf16 or fp32)")
    return SaParams(B, H, N, d, cfg.block_q, cfg.block_k, cfg.tau, cfg.tau_mode, cfg.max_keep, cfg.min_keep,
                    cfg.n_dense_prefix, cfg.scale, dt,
                    (FLAG_NO_RESIDUAL if cfg.no_residual else 0) | (FLAG_PAMA if cfg.proxy == PAMA else 0) |
                    (FLAG_FUSED if cfg.fused else 0))


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")


def kv_idx_cap(p: SaParams) -> int:
    c = lib.sparse_attn_kv_idx_cap(ctypes.byref(p))
    if c < 0:
        _check(c)
    return c


# sa_params fields a route is built for.  A forward must use the route with the
# same values (the header's contract); only SA_FLAG_NO_RESIDUAL, a forward-only
# switch, may differ.
_ROUTE_FIELDS = ("B", "H", "N", "d", "block_q", "block_k", "tau", "tau_mode", "max_keep", "min_keep",
                 "n_dense_prefix", "scale", "dtype")
_SHAPE_FIELDS = ("B", "H", "N", "d", "block_q", "block_k", "dtype")


def _params_diff(a: SaParams, b: SaParams, fields) -> list:
    diff = [f"{f} {getattr(a, f)} != {getattr(b, f)}" for f in fields if getattr(a, f) != getattr(b, f)]
    fa, fb = a.flags & ~FLAG_NO_RESIDUAL, b.flags & ~FLAG_NO_RESIDUAL
    if fa != fb:
        diff.append(f"routing flags 0x{fa:x} != 0x{fb:x}")
    return diff


def _check_out(name: str, t: torch.Tensor, like: torch.Tensor, dtype=None):
    """An out= tensor: same device and shape as `like`, contiguous, of `like`'s dtype (or `dtype`)."""
    want = like.dtype if dtype is None else dtype
    if not isinstance(t, torch.Tensor) or t.device != like.device or tuple(t.shape) != tuple(like.shape) \
            or t.dtype != want or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {want} tensor of shape {tuple(like.shape)} on {like.device}")


def route_sizes(p: SaParams, cap: int) -> list:
    arr = (ctypes.c_size_t * len(BUFFERS))()
    _check(lib.sparse_attn_route_sizes(ctypes.byref(p), cap, arr))
    return list(arr)


class Route:
    """Device buffers written by route() and read by forward()."""

    def __init__(self, p: SaParams, device, cap: int | None = None):
        self.params = SaParams.from_buffer_copy(p)
        self.cap = kv_idx_cap(p) if cap is None else cap
        sizes = route_sizes(p, self.cap)
        B, H, N, d = p.B, p.H, p.N, p.d
        self.n_qb = -(-N // p.block_q)
        self.n_kb = -(-N // p.block_k)
        words = -(-self.n_kb // 32)
        e = dict(device=device)
        self.kv_count = torch.empty((B, H, self.n_qb), dtype=torch.int32, **e)
        self.kv_idx = torch.empty((B, H, self.n_qb, self.cap), dtype=torch.int32, **e)
        self.kv_mask = torch.empty((B, H, self.n_qb, words), dtype=torch.int32, **e)
        self.q_mean = torch.empty((B, H, self.n_qb, d), dtype=torch.float32, **e)
        self.k_mean = torch.empty((B, H, self.n_kb, d), dtype=torch.float32, **e)
        self.v_mean = torch.empty((B, H, self.n_kb, d), dtype=torch.float32, **e)
        self.kv_split = torch.empty((B, H, 2, words, 64, d), dtype=torch.bfloat16, **e)
        self.row_stats = torch.empty((B, H, self.n_qb, 2), dtype=torch.float32, **e)
        self.cost = torch.empty((B, H, self.n_qb), dtype=torch.int32, **e)
        self.work_order = torch.empty((B * H * self.n_qb,), dtype=torch.int32, **e)
        self.k_bounds = torch.empty((B, H, words, 2), dtype=torch.float32, **e)
        for name, nbytes in zip(BUFFERS, sizes):
            t = getattr(self, name)
            if t.numel() * t.element_size() != nbytes:
                raise RuntimeError(f"route buffer {name}: {t.numel() * t.element_size()} bytes, library wants {nbytes}")
        self.c = SaRoute(*[getattr(self, n).data_ptr() for n in BUFFERS], self.cap)

    def check(self, p: SaParams, who: str, fields=_ROUTE_FIELDS):
        """ValueError unless this route was built for p (before anything is enqueued)."""
        diff = _params_diff(self.params, p, fields)
        if diff:
            raise ValueError(f"{who}: the route was built for other parameters ({'; '.join(diff)})")
        if self.cap < kv_idx_cap(p):
            raise ValueError(f"{who}: route kv_idx capacity {self.cap} < {kv_idx_cap(p)} needed")

    def mask(self) -> torch.Tensor:
        """Keep mask as bool [B, H, n_qb, n_kb] (unpacked from the bit words, on device)."""
        w = self.kv_mask.to(torch.int64) & 0xFFFFFFFF
        bits = torch.arange(32, device=w.device, dtype=torch.int64)
        m = ((w[..., :, None] >> bits) & 1).bool().flatten(-2)
        return m[..., : self.n_kb]


def route(q, k, v, cfg: Config, out: Route | None = None) -> Route:
    """sparse_attn_route: block routing; returns the route buffers."""
    _check_qkv(q, k, v)
    p = make_params(q, cfg)
    if out is not None:
        # reusable for new routing fields (tau, budget, mode) at the same shapes
        out.check(p, "route(out=...)", _SHAPE_FIELDS)
        if out.kv_count.device != q.device:
            raise ValueError("route(out=...): the route's buffers are on another device")
    rt = out if out is not None else Route(p, q.device)
    rt.params = SaParams.from_buffer_copy(p)
    _check(lib.sparse_attn_route(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(rt.c),
                                 _stream(q.device)))
    return rt


def forward(q, k, v, rt: Route, cfg: Config, out: torch.Tensor | None = None, lse: bool = False):
    """sparse_attn_forward: exact kept tiles plus dropped-block residual. Returns o or (o, lse)."""
    _check_qkv(q, k, v)
    p = make_params(q, cfg)
    rt.check(p, "forward")
    if out is not None:
        _check_out("out", out, q)
    o = out if out is not None else torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse else None
    _check(lib.sparse_attn_forward(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(rt.c),
                                   o.data_ptr(), L.data_ptr() if lse else None, _stream(q.device)))
    return (o, L) if lse else o


def dense_ref_gpu(q, k, v, block_q: int = 128, scale: float = 0.0, out: torch.Tensor | None = None,
                  lse: bool = False):
    """sparse_attn_dense_ref_gpu: dense softmax attention with the same kernels."""
    _check_qkv(q, k, v)
    p = make_params(q, Config(block_q=block_q, block_k=128, scale=scale))
    if out is not None:
        _check_out("out", out, q)
    o = out if out is not None else torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse else None
    _check(lib.sparse_attn_dense_ref_gpu(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         L.data_ptr() if lse else None, _stream(q.device)))
    return (o, L) if lse else o


def sparsepr_workspace_size(q, cfg: Config, probes_per_block: int) -> int:
    """sparse_attn_sparsepr_workspace_size: bytes of the probe-fitted residual's workspace."""
    p = make_params(q, cfg)
    n = ctypes.c_size_t()
    _check(lib.sparse_attn_sparsepr_workspace_size(ctypes.byref(p), probes_per_block, ctypes.byref(n)))
    return n.value


def forward_sparsepr(q, k, v, rt: Route, cfg: Config, probes_per_block: int = 2, rank: int = 8,
                     ridge: float = 1e-3, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """sparse_attn_forward_sparsepr: attention over the kept tokens, corrected by an
    affine map fitted on exact probe rows (in place of the block residual)."""
    _check_qkv(q, k, v)
    p = make_params(q, cfg)
    rt.check(p, "forward_sparsepr")
    n = sparsepr_workspace_size(q, cfg, probes_per_block)
    if workspace is not None and (workspace.device != q.device or workspace.dtype != torch.uint8
                                  or not workspace.is_contiguous() or workspace.numel() < n):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {n} bytes on {q.device}")
    if out is not None:
        _check_out("out", out, q)
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty_like(q)
    _check(lib.sparse_attn_forward_sparsepr(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            ctypes.byref(rt.c), probes_per_block, rank, ridge, ws.data_ptr(),
                                            ws.numel(), o.data_ptr(), _stream(q.device)))
    return o


def forward_sparsepr_static(q, k, v, rt: Route, cfg: Config, probes_per_block: int = 2, rank: int = 8,
                            ridge: float = 1e-3, out: torch.Tensor | None = None) -> torch.Tensor:
    """sparse_attn_forward_sparsepr_static: forward_sparsepr with its intermediates in
    the library's static per-GPU array (no workspace; the library allocates nothing).
    Calls that overlap on one GPU race; out= lets the caller allocate nothing either."""
    _check_qkv(q, k, v)
    p = make_params(q, cfg)
    rt.check(p, "forward_sparsepr_static")
    if out is not None:
        _check_out("out", out, q)
    o = out if out is not None else torch.empty_like(q)
    _check(lib.sparse_attn_forward_sparsepr_static(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                   ctypes.byref(rt.c), probes_per_block, rank, ridge,
                                                   o.data_ptr(), _stream(q.device)))
    return o


def hilbert_order(T: int, Hh: int, W: int) -> torch.Tensor:
    """sparse_attn_hilbert_order: int32 [T*Hh*W] (CPU), raster index of the token at
    each Hilbert curve position."""
    perm = torch.empty(T * Hh * W, dtype=torch.int32)
    _check(lib.sparse_attn_hilbert_order(T, Hh, W, ctypes.cast(perm.data_ptr(), ctypes.POINTER(ctypes.c_int32))))
    return perm


def permute_tokens(x: torch.Tensor, perm: torch.Tensor, n0: int = 0, inverse: bool = False,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """sparse_attn_permute_tokens: rows [n0, n0 + len(perm)) of x [B, H, N, d] gathered
    by perm (inverse=False) or scattered by it (inverse=True); other rows copied."""
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] device tensor")
    dt = {torch.bfloat16: SA_BF16, torch.float32: SA_F32}.get(x.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {x.dtype} (bf16 or fp32)")
    if perm.dtype != torch.int32 or perm.device != x.device or not perm.is_contiguous():
        raise ValueError("perm must be a contiguous int32 tensor on x's device")
    o = out if out is not None else torch.empty_like(x)
    if o.shape != x.shape or o.dtype != x.dtype or not o.is_contiguous():
        raise ValueError("out must match x")
    B, H, N, d = x.shape
    _check(lib.sparse_attn_permute_tokens(B, H, N, d, dt, n0, perm.numel(), perm.data_ptr() if perm.numel() else None,
                                          int(inverse), x.data_ptr(), o.data_ptr(), _stream(x.device)))
    return o


def status_string(s: int) -> str:
    return lib.sparse_attn_status_string(s).decode()


def last_error() -> str:
    return lib.sparse_attn_last_error().decode()


def dense_flops(B: int, H: int, N: int, d: int) -> float:
    """4 B H N^2 d: the flops of dense attention (QK^T and PV)."""
    return 4.0 * B * H * N * N * d


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
