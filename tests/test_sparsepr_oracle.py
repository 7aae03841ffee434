"""Pins of the probe-fitted residual oracle (SparsePR summary, section B) against
closed forms, a library least-squares routine and the algebra of projections."""
import numpy as np
import pytest

from oracle import sparse_attn_ref as R
from oracle import sparsepr as SP


def test_probe_rows_are_stratified_per_block():
    rows = SP.probe_rows(300, 128, 3)                     # blocks of 128, 128, 44 rows
    assert rows.tolist() == [21, 64, 106, 149, 192, 234, 263, 278, 292]
    for I in range(3):
        blk = rows[3 * I:3 * I + 3]
        assert ((blk >= I * 128) & (blk < min(300, (I + 1) * 128))).all()
    assert (np.diff(rows) > 0).all()


def test_fit_recovers_an_exactly_affine_low_rank_residual():
    """If R = b0 + X B0 has rank <= k, the fit returns b0 and B0 (tiny ridge) and
    the projection leaves every such correction unchanged: the corrected output
    equals O_s + b0 + O_s B0 on every row."""
    rng = np.random.default_rng(0)
    M, d, k = 200, 16, 3
    U = rng.standard_normal((d, k))
    W = rng.standard_normal((k, d))
    B0 = U @ W * 0.1                                      # rank k
    b0 = rng.standard_normal(k) @ W * 0.05                # inside the same row space
    X = rng.standard_normal((M, d))
    Rres = b0[None, :] + X @ B0
    b, B, Pk = SP.fit(X, Rres, ridge=1e-14, rank=k)
    np.testing.assert_allclose(B, B0, atol=1e-9)
    np.testing.assert_allclose(b, b0, atol=1e-9)
    Os = rng.standard_normal((50, d))
    out = SP.correct(Os, np.zeros((0, d)), np.zeros(0, dtype=np.int64), b, B, Pk)
    np.testing.assert_allclose(out, Os + b0 + Os @ B0, atol=1e-9)


def test_ridge_matches_augmented_least_squares():
    rng = np.random.default_rng(1)
    M, d = 60, 8
    X, Rres = rng.standard_normal((M, d)), rng.standard_normal((M, d))
    ridge = 0.3
    b, B, _ = SP.fit(X, Rres, ridge=ridge, rank=d)
    Xc, Rc = X - X.mean(0), Rres - Rres.mean(0)
    lam = ridge * np.trace(Xc.T @ Xc) / d
    A = np.vstack([Xc, np.sqrt(lam) * np.eye(d)])
    Y = np.vstack([Rc, np.zeros((d, d))])
    B_ls = np.linalg.lstsq(A, Y, rcond=None)[0]
    np.testing.assert_allclose(B, B_ls, atol=1e-12)
    np.testing.assert_allclose(b, Rres.mean(0) - X.mean(0) @ B_ls, atol=1e-12)


@pytest.mark.parametrize("k", [1, 4, 8])
def test_projection_is_symmetric_idempotent_of_rank_k(k):
    rng = np.random.default_rng(k)
    X, Rres = rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    _, _, Pk = SP.fit(X, Rres, ridge=1e-3, rank=k)
    np.testing.assert_allclose(Pk, Pk.T, atol=1e-13)
    np.testing.assert_allclose(Pk @ Pk, Pk, atol=1e-12)
    assert abs(np.trace(Pk) - k) < 1e-12
    # it spans the leading right singular vectors: their residual energy is kept
    _, s, _ = np.linalg.svd(Rres, full_matrices=False)
    np.testing.assert_allclose(np.linalg.norm(Rres @ Pk) ** 2, (s[:k] ** 2).sum(), rtol=1e-12)


def test_everything_kept_needs_no_correction():
    rng = np.random.default_rng(4)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = R.RouteParams(32, 16, 0.0)
    mask = np.ones((3, 6), dtype=bool)
    out, (Os, probes, Od, b, B, Pk) = SP.sparsepr_ref(q, k, v, mask, p, per_block=4, rank=4, ridge=1e-3)
    dense, _ = R.dense_ref(q, k, v)
    np.testing.assert_allclose(Os, dense, atol=1e-12)
    np.testing.assert_allclose(out, dense, atol=1e-10)


def test_probe_rows_take_exact_values():
    rng = np.random.default_rng(5)
    N, d = 130, 8
    q, k, v = (rng.standard_normal((N, d)) * s for s in (2.0, 1.0, 1.0))
    p = R.RouteParams(64, 16, 0.3)
    mask = R.route_ref(q, k, p).mask
    out, (Os, probes, Od, *_ ) = SP.sparsepr_ref(q, k, v, mask, p, per_block=5, rank=4, ridge=1e-2)
    dense, _ = R.dense_ref(q, k, v)
    np.testing.assert_allclose(out[probes], dense[probes], atol=1e-12)
