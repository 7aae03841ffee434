"""Token reordering: the oracle's Hilbert order against the properties that
define a Hilbert path, the library's host order against the oracle, and the
host checks of the permutation entry point (no GPU needed here)."""
import ctypes

import numpy as np
import pytest

from oracle import reorder as RO


def grid_points(T, Hh, W, perm):
    return np.stack([perm // (Hh * W), (perm // W) % Hh, perm % W], axis=1)


@pytest.mark.parametrize("b", [1, 2, 3])
def test_oracle_full_cube_is_a_unit_step_path_from_the_origin(b):
    n = 1 << b
    perm = RO.hilbert_order(n, n, n)
    assert sorted(perm.tolist()) == list(range(n ** 3))
    pts = grid_points(n, n, n, perm)
    assert (pts[0] == 0).all()
    steps = np.abs(np.diff(pts, axis=0)).sum(axis=1)
    assert (steps == 1).all()


def test_oracle_order_one_curve_is_the_reflected_gray_code():
    # J. Skilling, "Programming the Hilbert curve" (2004): with one bit plane the
    # transposed form of index i is i itself, whose Gray decoding gives the axes,
    # first axis most significant; the curve on the 2x2x2 cube is therefore the
    # binary reflected Gray code (a different unit-step path from the origin,
    # e.g. (0,0,0) (0,0,1) (0,1,1) (1,1,1) ..., fails here)
    pts = grid_points(2, 2, 2, RO.hilbert_order(2, 2, 2))
    gray = [(i ^ (i >> 1)) for i in range(8)]
    want = np.array([[(g >> 2) & 1, (g >> 1) & 1, g & 1] for g in gray])
    assert (pts == want).all()


@pytest.mark.parametrize("b", [2, 3])
def test_oracle_curve_fills_aligned_subcubes_in_turn(b):
    # self-similarity of a Hilbert curve: every run of 8^k consecutive points
    # fills one aligned sub-cube of side 2^k (a snake or other unit-step path
    # through the cube does not)
    n = 1 << b
    pts = grid_points(n, n, n, RO.hilbert_order(n, n, n))
    for k in range(1, b):
        run, side = 8 ** k, 1 << k
        for s in range(0, n ** 3, run):
            corner = pts[s:s + run] // side
            assert (corner == corner[0]).all(), (k, s)
            assert len({tuple(p) for p in pts[s:s + run] % side}) == run


def test_oracle_index_is_a_bijection_on_the_cube():
    b = 3
    idx = sorted(RO.hilbert_index(t, y, x, b) for t in range(8) for y in range(8) for x in range(8))
    assert idx == list(range(512))


@pytest.mark.parametrize("grid", [(1, 1, 1), (1, 1, 7), (3, 5, 7), (4, 8, 30), (2, 9, 3)])
def test_oracle_ragged_grid_is_a_permutation(grid):
    perm = RO.hilbert_order(*grid)
    assert sorted(perm.tolist()) == list(range(int(np.prod(grid))))


def test_oracle_ragged_grid_follows_the_cube_walk():
    # the grid's order is the cube's walk with the points outside the grid removed
    cube = RO.hilbert_order(8, 8, 8)
    pts = grid_points(8, 8, 8, cube)
    inside = (pts[:, 0] < 3) & (pts[:, 1] < 5) & (pts[:, 2] < 7)
    want = pts[inside]
    got = grid_points(3, 5, 7, RO.hilbert_order(3, 5, 7))
    assert (got == want).all()


def test_oracle_permute_rows_definition_and_round_trip():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 20, 4))
    perm = rng.permutation(12).astype(np.int32)
    g = RO.permute_rows(x, perm, n0=5)
    assert (g[..., :5, :] == x[..., :5, :]).all() and (g[..., 17:, :] == x[..., 17:, :]).all()
    for i in range(12):
        assert (g[..., 5 + i, :] == x[..., 5 + perm[i], :]).all()
    back = RO.permute_rows(g, perm, n0=5, inverse=True)
    assert (back == x).all()


# ----------------------------------------------------------------- library, host side
sa = pytest.importorskip("free_block_sparse_route_amd")


@pytest.mark.parametrize("grid", [(1, 1, 1), (2, 2, 2), (3, 5, 7), (4, 8, 30), (1, 1, 9), (8, 8, 8), (5, 17, 11)])
def test_library_hilbert_order_equals_oracle(grid):
    assert (sa.hilbert_order(*grid).numpy() == RO.hilbert_order(*grid)).all()


def test_library_hilbert_order_hunyuan_grid():
    grid = (33, 45, 80)
    got = sa.hilbert_order(*grid).numpy()
    assert sorted(got.tolist()) == list(range(int(np.prod(grid))))
    # spot check against the oracle index: curve positions are increasing
    b = RO.cube_bits(*grid)
    pts = grid_points(*grid, got[::997])
    idx = [RO.hilbert_index(*p, b) for p in pts]
    assert all(a < c for a, c in zip(idx, idx[1:]))


def test_library_hilbert_order_errors():
    lib = sa.binding.lib
    buf = (ctypes.c_int32 * 8)()
    assert lib.sparse_attn_hilbert_order(0, 2, 2, buf) == sa.binding.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_hilbert_order(2, 2, 2, None) == sa.binding.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_hilbert_order(1, 1, 513, buf) == sa.binding.SA_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    (dict(B=0), -1), (dict(d=96), -2), (dict(dtype=5), -1), (dict(n0=-1), -1), (dict(n_perm=11), -1),
    (dict(n0=4, n_perm=7), -1), (dict(inverse=2), -1), (dict(same=True), -1), (dict(perm=None), -1),
])
def test_permute_rejects_bad_arguments_before_launch(args, status):
    lib = sa.binding.lib
    a = dict(B=1, H=1, N=10, d=64, dtype=0, n0=0, n_perm=10, perm=1, inverse=0, same=False)
    a.update(args)
    inp, out = 0x1000, (0x1000 if a["same"] else 0x2000)   # never dereferenced: rejected first
    r = lib.sparse_attn_permute_tokens(a["B"], a["H"], a["N"], a["d"], a["dtype"], a["n0"], a["n_perm"],
                                       a["perm"] and 0x3000, a["inverse"], inp, out, None)
    assert r == status, sa.last_error()
