"""Oracle of token reordering: the 3D Hilbert order of a video token grid and
the row permutation that applies it.  TEST INFRASTRUCTURE ONLY (tests, smoke
check, benchmark CPU baseline); independent of the HIP library.

DFSAttn abstract: tokens are reordered along a 3D Hilbert curve before blocking,
so that a block of consecutive tokens is compact in space and time.

Curve: J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707
(2004), in its coordinates-to-index direction, one point at a time in plain
Python: the inverse undo of the excess work over the bit planes (high to low),
then the Gray encoding, give the curve's transposed form; the index is its bit
interleave, most significant plane first, axes (t, y, x).  The order of a
T x Hh x W grid is the stable sort of its raster tokens by that index on the
enclosing 2^b cube, b = max(1, ceil(log2(max side))).

Pins (tests/test_reorder.py): on full cubes consecutive positions are face
neighbours (the defining property of a Hilbert path) and the walk starts at the
origin; on ragged grids the order is a bijection; the row permutation is
checked against its definition and its round trip.
"""
from __future__ import annotations

import numpy as np


def hilbert_index(t: int, y: int, x: int, b: int) -> int:
    """Index of the point (t, y, x) on the 2^b cube."""
    X = [int(t), int(y), int(x)]
    Q = 1 << (b - 1)
    while Q > 1:                                   # inverse undo, high planes first
        P = Q - 1
        for i in range(3):
            if X[i] & Q:
                X[0] ^= P                          # invert the low bits of X[0]
            else:
                s = (X[0] ^ X[i]) & P              # exchange the low bits of X[0] and X[i]
                X[0] ^= s
                X[i] ^= s
        Q >>= 1
    X[1] ^= X[0]                                   # Gray encode
    X[2] ^= X[1]
    s = 0
    Q = 1 << (b - 1)
    while Q > 1:
        if X[2] & Q:
            s ^= Q - 1
        Q >>= 1
    X = [v ^ s for v in X]
    h = 0
    for p in range(b - 1, -1, -1):                 # interleave, msb plane first
        for i in range(3):
            h = (h << 1) | ((X[i] >> p) & 1)
    return h


def cube_bits(T: int, Hh: int, W: int) -> int:
    side = max(T, Hh, W)
    b = 1
    while (1 << b) < side:
        b += 1
    return b


def hilbert_order(T: int, Hh: int, W: int) -> np.ndarray:
    """perm[i] = raster index t*Hh*W + y*W + x of the token at curve position i."""
    b = cube_bits(T, Hh, W)
    keys = []
    for t in range(T):
        for y in range(Hh):
            for x in range(W):
                keys.append(hilbert_index(t, y, x, b))
    return np.argsort(np.asarray(keys, dtype=np.int64), kind="stable").astype(np.int32)


def permute_rows(x: np.ndarray, perm: np.ndarray, n0: int = 0, inverse: bool = False) -> np.ndarray:
    """Rows [n0, n0 + len(perm)) of x [..., N, d]: gather out[n0+i] = x[n0+perm[i]],
    or scatter out[n0+perm[i]] = x[n0+i]; other rows copied."""
    out = x.copy()
    n = len(perm)
    seg = np.arange(n0, n0 + n)
    if inverse:
        out[..., n0 + perm, :] = x[..., seg, :]
    else:
        out[..., seg, :] = x[..., n0 + perm, :]
    return out
