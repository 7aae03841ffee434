"""Seeded synthetic Q/K/V shaped like video-DiT attention layers.

This module is input data only. It holds none of the attention method's
arithmetic (no pooling, scores, selection or softmax); both the CPU oracle and
the GPU path take the tensors it returns as their inputs.

Token grids and per-config constants follow the workloads of the
block-sparse video attention problem statement (Wan-1.3B 480p, Wan-14B 720p,
HunyuanVideo 720p with a text prefix, a stress case with per-head query
scales).  The structure is the one those workloads describe:

  k_j = P e(pos_j) + 0.3 n_j,   q_i = s (P e(pos_i) + 0.3 n_i),   v ~ N(0, 1)

where e is a 3D sinusoidal position embedding with 24 dimensions per axis
(t, h, w), P is a seeded Gaussian 72 -> d projection with N(0, 1/72) entries,
n is independent standard normal noise for q and for k, and the keys of the
first 16 raster tokens are scaled by 3 (attention sinks).  The constants the
workload description leaves open are fixed here once and named:
EMB_BASE, NOISE, SINK_TOKENS, SINK_SCALE, the per-config query scale s.

Token reordering along a 3D Hilbert curve (DFSAttn abstract, "Hilbert
curve-based token reordering") is input preparation and lives here as well:
it permutes tokens before blocking and never changes any value.

Seeds: numpy SeedSequence((cfg_id, b, h)); the stress case draws its per-head
query scales from SeedSequence((cfg_id, 7)).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np

EMB_DIMS_PER_AXIS = 24          # 12 frequencies x (sin, cos)
EMB_BASE = 10000.0              # sinusoid frequency base
NOISE = 0.3                     # noise amplitude of q and k
SINK_TOKENS = 16                # raster tokens whose keys are attention sinks
SINK_SCALE = 3.0
STRESS_SCALE_RANGE = (1.0, 12.0)
STRESS_SCALE_STREAM = 7         # SeedSequence((cfg_id, 7)) draws stress query scales


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer shape with its routing knobs."""
    name: str
    cfg_id: int
    B: int
    H: int
    d: int
    grid: tuple            # (T, Hh, W) video token grid
    block_q: int
    block_k: int
    tau: float
    dtype: str             # "bf16" or "f32"
    qscale: float | None   # None => per-head draw from STRESS_SCALE_RANGE
    max_keep_frac: float = 0.0   # top-k budget as a fraction of KV blocks (0 = no cap)
    n_text: int = 0              # dense-attended text tokens placed before the video tokens
    hilbert: bool = False        # reorder video tokens along a 3D Hilbert curve

    @property
    def n_video(self) -> int:
        T, Hh, W = self.grid
        return T * Hh * W

    @property
    def N(self) -> int:
        return self.n_text + self.n_video

    @property
    def n_qb(self) -> int:
        return -(-self.N // self.block_q)

    @property
    def n_kb(self) -> int:
        return -(-self.N // self.block_k)

    @property
    def max_keep(self) -> int:
        return int(math.floor(self.max_keep_frac * self.n_kb)) if self.max_keep_frac > 0 else 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 64, (16, 16, 16), 64, 64, 0.02, "f32", 4.0),
    "wan1.3b": Workload("wan1.3b", 1, 1, 12, 128, (21, 30, 52), 128, 128, 0.01, "bf16", 6.0),
    "wan14b": Workload("wan14b", 2, 1, 40, 128, (21, 45, 80), 128, 64, 0.003, "bf16", 6.0,
                       max_keep_frac=0.25),
    "hunyuan": Workload("hunyuan", 3, 1, 24, 128, (33, 45, 80), 128, 128, 0.01, "bf16", 6.0,
                        n_text=256, hilbert=True),
    "stress": Workload("stress", 4, 2, 24, 128, (33, 45, 80), 128, 128, 0.05, "bf16", None),
}
WAN14B_TAU_SWEEP = (0.003, 0.01, 0.03)


def small(name: str, B: int, H: int, d: int, grid: tuple, block_q: int, block_k: int,
          tau: float, dtype: str = "bf16", qscale: float = 6.0, cfg_id: int = 100,
          **kw) -> Workload:
    """A reduced workload with the same generator, for tests."""
    return Workload(name, cfg_id, B, H, d, tuple(grid), block_q, block_k, tau, dtype, qscale, **kw)


# ----------------------------------------------------------------------------- positions
def raster_positions(grid: tuple) -> np.ndarray:
    """(t, y, x) integer coordinates of the video tokens in raster order, [N, 3]."""
    T, Hh, W = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


def sinusoid_embedding(pos: np.ndarray) -> np.ndarray:
    """3D sinusoidal embedding, [N, 72] float64: per axis [sin(p w_k), cos(p w_k)], k < 12,
    with w_k = EMB_BASE ** (-2k / 24)."""
    half = EMB_DIMS_PER_AXIS // 2
    w = EMB_BASE ** (-2.0 * np.arange(half) / EMB_DIMS_PER_AXIS)
    parts = []
    for a in range(3):
        ang = pos[:, a:a + 1].astype(np.float64) * w[None, :]
        parts += [np.sin(ang), np.cos(ang)]
    # axis-major: [sin_t, cos_t, sin_h, cos_h, sin_w, cos_w]
    return np.concatenate(parts, axis=1)


def hilbert_index_3d(pos: np.ndarray, bits: int) -> np.ndarray:
    """Index of integer points along a 3D Hilbert curve on the 2**bits cube.

    Written from J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc.
    707 (2004): coordinates are turned into the curve's "transposed" form by an
    inverse-undo pass over the bit planes followed by a Gray encoding, and the
    index is the bit interleave of that form, most significant plane first.
    Vectorised over points.  pos: [N, 3] non-negative ints < 2**bits.
    """
    X = [pos[:, i].astype(np.int64).copy() for i in range(3)]
    n = 3
    top = 1 << (bits - 1)
    # inverse undo of the excess work
    Q = top
    while Q > 1:
        P = Q - 1
        for i in range(n):
            hit = (X[i] & Q) != 0
            # where the bit is set: invert the low bits of X[0]
            X0_inv = X[0] ^ P
            # otherwise: exchange the low bits of X[0] and X[i]
            t = (X[0] ^ X[i]) & P
            X0_swp = X[0] ^ t
            Xi_swp = X[i] ^ t
            if i == 0:
                X[0] = np.where(hit, X0_inv, X0_swp)  # for i == 0 the exchange is a no-op
            else:
                X[0], X[i] = np.where(hit, X0_inv, X0_swp), np.where(hit, X[i], Xi_swp)
        Q >>= 1
    # Gray encode
    for i in range(1, n):
        X[i] = X[i] ^ X[i - 1]
    t = np.zeros_like(X[0])
    Q = top
    while Q > 1:
        t = np.where((X[n - 1] & Q) != 0, t ^ (Q - 1), t)
        Q >>= 1
    for i in range(n):
        X[i] = X[i] ^ t
    # interleave: plane b (msb first), axis 0..n-1
    idx = np.zeros_like(X[0])
    for b in range(bits - 1, -1, -1):
        for i in range(n):
            idx = (idx << 1) | ((X[i] >> b) & 1)
    return idx


def hilbert_permutation(grid: tuple) -> np.ndarray:
    """perm such that video_tokens[perm] is in Hilbert order (stable sort of the index
    on the enclosing power-of-two cube)."""
    bits = max(1, int(math.ceil(math.log2(max(grid)))))
    idx = hilbert_index_3d(raster_positions(grid), bits)
    return np.argsort(idx, kind="stable")


# ----------------------------------------------------------------------------- heads
def query_scales(w: Workload) -> np.ndarray:
    """Per-head query scale s, [H]."""
    if w.qscale is not None:
        return np.full(w.H, float(w.qscale))
    rng = np.random.default_rng(np.random.SeedSequence((w.cfg_id, STRESS_SCALE_STREAM)))
    lo, hi = STRESS_SCALE_RANGE
    return rng.uniform(lo, hi, size=w.H)


class _Shared:
    """Position embedding and permutation shared by every head of one workload."""

    def __init__(self, w: Workload):
        self.emb = sinusoid_embedding(raster_positions(w.grid))          # [Nv, 72]
        self.perm = hilbert_permutation(w.grid) if w.hilbert else None
        self.scales = query_scales(w)


def head_qkv(w: Workload, b: int, h: int, shared: _Shared | None = None):
    """q, k, v for one (b, h) as float64 arrays [N, d] (before any dtype cast)."""
    sh = shared or _Shared(w)
    rng = np.random.default_rng(np.random.SeedSequence((w.cfg_id, b, h)))
    d, Nv = w.d, w.n_video
    P = rng.standard_normal((sh.emb.shape[1], d)) / math.sqrt(sh.emb.shape[1])
    base = sh.emb @ P                                                    # [Nv, d]
    k = base + NOISE * rng.standard_normal((Nv, d))
    q = sh.scales[h] * (base + NOISE * rng.standard_normal((Nv, d)))
    v = rng.standard_normal((Nv, d))
    k[:SINK_TOKENS] *= SINK_SCALE                                        # raster tokens 0..15
    if sh.perm is not None:
        q, k, v = q[sh.perm], k[sh.perm], v[sh.perm]
    if w.n_text:
        tq = rng.standard_normal((w.n_text, d))
        tk = rng.standard_normal((w.n_text, d))
        tv = rng.standard_normal((w.n_text, d))
        q = np.concatenate([tq, q]); k = np.concatenate([tk, k]); v = np.concatenate([tv, v])
    return q, k, v


def iter_heads(w: Workload) -> Iterator[tuple]:
    sh = _Shared(w)
    for b in range(w.B):
        for h in range(w.H):
            yield b, h, head_qkv(w, b, h, sh)


def make_qkv(w: Workload, device: str = "cpu", heads: list | None = None, workers: int | None = None):
    """Q, K, V as torch tensors [B, H, N, d] in the workload dtype (bf16 by torch's cast
    from float64, or float32), built one head at a time (heads in parallel threads; each
    head has its own seed, so the result does not depend on scheduling).  `heads`
    optionally restricts to a list of (b, h); others stay zero."""
    import concurrent.futures as cf
    import os

    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = (w.B, w.H, w.N, w.d)
    out = [torch.zeros(shape, dtype=tdt) for _ in range(3)]
    sh = _Shared(w)
    todo = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        for dst, a in zip(out, head_qkv(w, b, h, sh)):
            dst[b, h].copy_(torch.from_numpy(a).to(tdt))

    n = workers or min(16, len(os.sched_getaffinity(0)), max(1, len(todo)))
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, todo))
    if device != "cpu":
        out = [t.to(device) for t in out]
    return tuple(out)
