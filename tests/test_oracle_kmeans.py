"""Pins for the oracle's Lloyd k-means (clustering of queries and of keys,
each in its own space: gist.science Technical Summary, Core Mechanisms,
Bidirectional Semantic Clustering).  The reading "Lloyd, fixed iterations,
ties to the lowest index, empty clusters keep their centroid" is pinned to
scipy's independent kmeans2, which implements exactly that loop."""
import warnings

import numpy as np
import pytest

from oracle import muse_oracle as mo


def _scipy_kmeans(X, init, iters):
    from scipy.cluster.vq import kmeans2
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        cb, lab = kmeans2(X, X[init].copy(), iter=iters, minit="matrix", missing="warn")
    return lab, cb


@pytest.mark.parametrize("trial", range(40))
def test_kmeans_matches_scipy(trial):
    rng = np.random.default_rng(1000 + trial)
    n = int(rng.integers(20, 300))
    D = int(rng.integers(1, 9))
    C = int(rng.integers(1, min(n, 24) + 1))
    iters = int(rng.integers(1, 12))
    if trial % 4 == 0:
        # few distinct values: exact distance ties and empty clusters
        X = rng.integers(-2, 3, size=(n, D)).astype(np.float64)
        X[: n // 2] = X[0]
    else:
        X = rng.standard_normal((n, D))
    init = rng.choice(n, C, replace=False)
    if trial % 4 == 0:
        # distinct starting indices may still hold equal points: scipy and
        # the oracle both start from the same coordinates
        pass
    lab, mu = mo.kmeans(X, C, iters, init)
    slab, smu = _scipy_kmeans(X, init, iters)
    assert np.array_equal(lab, slab)
    np.testing.assert_allclose(mu, smu, rtol=0, atol=1e-12)


def test_kmeans_fixed_point_invariants():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((500, 6))
    init = rng.choice(500, 12, replace=False)
    lab, mu, hist = mo.kmeans(X, 12, 8, init, history=True)
    prev = X[init]
    for labels_t, mu_t in hist:
        d = ((X[:, None, :] - prev[None]) ** 2).sum(-1)
        assert np.array_equal(labels_t, np.argmin(d, axis=1))
        for c in range(12):
            mem = X[labels_t == c]
            want = mem.mean(0) if len(mem) else prev[c]
            np.testing.assert_allclose(mu_t[c], want, atol=1e-13)
        prev = mu_t
    assert np.array_equal(lab, hist[-1][0])


def test_kmeans_recovers_separated_mixture():
    rng = np.random.default_rng(3)
    C, D, n = 8, 16, 800
    centres = rng.standard_normal((C, D)) * 10
    truth = rng.integers(0, C, n)
    X = centres[truth] + 0.1 * rng.standard_normal((n, D))
    init = np.array([np.nonzero(truth == c)[0][0] for c in range(C)])
    lab, mu = mo.kmeans(X, C, 5, init)
    assert np.array_equal(lab, truth)
    for c in range(C):
        np.testing.assert_allclose(mu[c], X[truth == c].mean(0), atol=1e-12)


def test_default_init_is_distinct_and_in_range():
    for n, C in [(1, 1), (5, 5), (1000, 16), (1024, 128), (17, 16)]:
        ii = mo.default_init(n, C)
        assert len(set(ii.tolist())) == C and ii.min() >= 0 and ii.max() < n


def test_default_init_is_floor_of_c_n_over_C():
    """The default starting points are evenly spread, floor(c n / C); the
    values below are written out by hand at sizes where the rounding order
    matters (c * floor(n / C) gives 0, 2, 4, 6 for n = 10, C = 4)."""
    assert mo.default_init(10, 4).tolist() == [0, 2, 5, 7]
    assert mo.default_init(1000, 7).tolist() == [0, 142, 285, 428, 571, 714, 857]
    assert mo.default_init(5, 3).tolist() == [0, 1, 3]
    assert mo.default_init(4, 4).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("trial", range(12))
def test_warm_started_kmeans_matches_scipy_from_the_same_centroids(trial):
    """A warm start continues Lloyd from given centroids: scipy's kmeans2
    with those centroids as its starting matrix agrees, including from
    centroids that are no data point and with clusters that end empty."""
    rng = np.random.default_rng(2000 + trial)
    n, D, C = int(rng.integers(30, 200)), int(rng.integers(1, 7)), int(rng.integers(2, 12))
    X = rng.standard_normal((n, D))
    mu0 = rng.standard_normal((C, D)) * (3.0 if trial % 3 == 0 else 1.0)
    iters = int(rng.integers(1, 6))
    lab, mu = mo.kmeans_from(X, mu0, iters)
    from scipy.cluster.vq import kmeans2
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        smu, slab = kmeans2(X, mu0.copy(), iter=iters, minit="matrix", missing="warn")
    assert np.array_equal(lab, slab)
    np.testing.assert_allclose(mu, smu, rtol=0, atol=1e-12)


def test_warm_start_continues_a_clustering():
    """T1 iterations, then T2 more from the resulting centroids, is T1 + T2
    iterations from the start."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((400, 5))
    init = rng.choice(400, 9, replace=False)
    _, mu1 = mo.kmeans(X, 9, 3, init)
    lab2, mu2 = mo.kmeans_from(X, mu1, 4)
    lab7, mu7 = mo.kmeans(X, 9, 7, init)
    assert np.array_equal(lab2, lab7)
    np.testing.assert_array_equal(mu2, mu7)
