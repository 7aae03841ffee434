"""Seeded input generator: shapes, determinism, structure, Hilbert order."""
import math

import numpy as np
import pytest

from workloads import synth as S


def test_workload_sizes():
    w = S.WORKLOADS
    assert (w["tiny"].N, w["tiny"].n_qb, w["tiny"].n_kb) == (4096, 64, 64)
    assert (w["wan1.3b"].N, w["wan1.3b"].n_qb, w["wan1.3b"].n_kb) == (32760, 256, 256)
    assert (w["wan14b"].N, w["wan14b"].n_qb, w["wan14b"].n_kb) == (75600, 591, 1182)
    assert w["wan14b"].max_keep == 295
    assert (w["hunyuan"].N, w["hunyuan"].n_qb) == (119056, 931)
    assert (w["stress"].N, w["stress"].n_qb, w["stress"].B) == (118800, 929, 2)


def test_hilbert_curve_is_a_unit_step_path():
    """On a full 2^p cube, consecutive Hilbert indices are face neighbours and the
    index is a bijection onto 0..8^p-1."""
    for bits in (1, 2, 3, 4):
        n = 1 << bits
        pos = S.raster_positions((n, n, n))
        idx = S.hilbert_index_3d(pos, bits)
        assert np.array_equal(np.sort(idx), np.arange(n ** 3))
        path = pos[np.argsort(idx)]
        steps = np.abs(np.diff(path, axis=0)).sum(axis=1)
        assert (steps == 1).all()
        assert (path[0] == 0).all()


def test_hilbert_permutation_on_ragged_grid():
    grid = (3, 5, 7)
    perm = S.hilbert_permutation(grid)
    assert np.array_equal(np.sort(perm), np.arange(3 * 5 * 7))
    pos = S.raster_positions(grid)[perm]
    # locality: most consecutive tokens stay close
    steps = np.abs(np.diff(pos, axis=0)).sum(axis=1)
    assert np.median(steps) == 1


def test_generator_is_deterministic_and_structured():
    w = S.small("t", 1, 2, 16, (4, 4, 8), 16, 16, 0.05)
    a = S.head_qkv(w, 0, 1)
    b = S.head_qkv(w, 0, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = S.head_qkv(w, 0, 0)
    assert not np.array_equal(a[0], c[0])
    q, k, v = a
    assert q.shape == k.shape == v.shape == (128, 16)
    # sinks: the first 16 raster keys are 3x larger on average
    assert np.linalg.norm(k[:16]) > 2.0 * np.linalg.norm(k[16:32])
    # q and k share the positional projection: strongly correlated per token
    cor = np.corrcoef(q.ravel(), k.ravel())[0, 1]
    assert cor > 0.3


def test_text_prefix_and_reorder():
    w = S.small("t", 1, 1, 8, (2, 4, 4), 16, 16, 0.05, n_text=16, hilbert=True)
    q, k, v = S.head_qkv(w, 0, 0)
    assert q.shape == (48, 8)
    w2 = w.with_(hilbert=False)
    q2, k2, v2 = S.head_qkv(w2, 0, 0)
    assert np.array_equal(q[:16], q2[:16])                      # text tokens in front, unpermuted
    perm = S.hilbert_permutation(w.grid)
    assert np.array_equal(q[16:], q2[16:][perm])


def test_stress_scales_in_range():
    s = S.query_scales(S.WORKLOADS["stress"])
    assert s.shape == (24,) and s.min() >= 1.0 and s.max() <= 12.0 and s.std() > 1.0


def test_make_qkv_bf16_roundtrip():
    torch = pytest.importorskip("torch")
    w = S.small("t", 1, 2, 16, (2, 4, 8), 16, 16, 0.05)
    Q, K, V = S.make_qkv(w)
    assert Q.dtype == torch.bfloat16 and Q.shape == (1, 2, 64, 16)
    q, k, v = S.head_qkv(w, 0, 1)
    assert torch.equal(Q[0, 1], torch.from_numpy(q).to(torch.bfloat16))
