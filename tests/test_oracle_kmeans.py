"""Pins of oracle.kmeans: brute force on tiny inputs, Lloyd monotonicity, exact
recovery of noise-free prototypes, tie and empty-cluster rules."""
import itertools

import numpy as np
import pytest

from oracle import kmeans as km


def test_distances_equal_python_loop():
    rng = np.random.default_rng(0)
    y = rng.standard_normal((7, 5)).astype(np.float32)
    c = rng.standard_normal((3, 5)).astype(np.float32)
    w = rng.uniform(0.1, 3, 5).astype(np.float32)
    d = km.sq_distances(y, c, w)
    for i in range(7):
        for j in range(3):
            ref = 0.0
            for k in range(5):
                diff = float(y[i, k]) - float(c[j, k])
                ref += float(w[k]) * diff * diff
            assert d[i, j] == pytest.approx(ref, rel=1e-15)


def test_strided_init():
    y = np.arange(40, dtype=np.float32).reshape(10, 4)
    c = km.init_centroids(y, 3)        # floor(10 / 3) = 3 -> rows 0, 3, 6
    assert np.array_equal(c[:, 0], [0, 12, 24])


def test_ties_go_to_lowest_index():
    y = np.array([[0.0, 0.0], [2.0, 0.0]], np.float32)
    c = np.array([[1.0, 1.0], [1.0, -1.0], [1.0, 1.0]], np.float32)  # all equidistant
    labels, _ = km.assign(y, c)
    assert labels.tolist() == [0, 0]


def test_empty_cluster_keeps_centroid():
    y = np.array([[0.0], [0.1], [10.0]], np.float32)
    c = np.array([[0.0], [10.0], [100.0]], np.float32)
    labels, _ = km.assign(y, c)
    new, counts = km.update(y, labels, c)
    assert counts.tolist() == [2, 1, 0]
    assert new[2, 0] == np.float32(100.0)
    assert new[0, 0] == np.float32(np.float64(np.float32(0.1)) / 2)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    """N <= 8, C in {2, 3}: every assign label is the true argmin; the final
    objective is no worse than the initial one and no better than the global
    optimum over all C^N assignments (with means as centroids)."""
    rng = np.random.default_rng(seed)
    n, d, c = 7, 2, 2 + seed % 2
    y = rng.standard_normal((n, d)).astype(np.float32)
    w = None if seed % 3 else rng.uniform(0.5, 2.0, d).astype(np.float32)
    tr = km.kmeans(y, c, iters=10, w=w)
    for cin, lab in zip(tr.centroids_in, tr.labels_iter):
        for i in range(n):
            dist = [sum((1.0 if w is None else float(w[k])) * (float(y[i, k]) - float(cin[j, k])) ** 2
                        for k in range(d)) for j in range(c)]
            assert lab[i] == int(np.argmin(dist))
    j_final = tr.j_after_update[-1]
    j_init = km.objective(km.sq_distances(y, km.init_centroids(y, c), w),
                          km.assign(y, km.init_centroids(y, c), w)[0])
    best = np.inf
    y64 = y.astype(np.float64)
    wk = np.ones(d) if w is None else w.astype(np.float64)
    for lab in itertools.product(range(c), repeat=n):
        lab = np.array(lab)
        tot = 0.0
        for j in range(c):
            m = y64[lab == j]
            if len(m):
                tot += float((((m - m.mean(0)) ** 2) * wk).sum())
        best = min(best, tot)
    assert j_final <= j_init * (1 + 1e-6)
    assert j_final >= best * (1 - 1e-6)


@pytest.mark.parametrize("weighted", [False, True])
def test_lloyd_objective_never_increases(weighted):
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((400, 16)) * rng.uniform(0.1, 30, 16)).astype(np.float32)
    w = rng.uniform(0.2, 5, 16).astype(np.float32) if weighted else None
    tr = km.kmeans(y, 12, iters=10, w=w)
    seq = []
    for a, u in zip(tr.j_after_assign, tr.j_after_update):
        seq += [a, u]
    for prev, nxt in zip(seq, seq[1:]):
        # centroids are rounded to float32, hence a tiny relative slack
        assert nxt <= prev * (1 + 1e-6)


def test_noise_free_prototypes_recovered_exactly():
    rng = np.random.default_rng(4)
    c_true, d = 8, 16
    protos = np.round(rng.standard_normal((c_true, d)) * 8).astype(np.float32)
    reps = 5
    # arrange so that the strided init (stride N / C = reps) hits every prototype
    y = np.repeat(protos, reps, axis=0)
    tr = km.kmeans(y, c_true, iters=10)
    assert np.array_equal(tr.centroids, protos)
    assert np.array_equal(tr.labels, np.repeat(np.arange(c_true), reps))
    assert tr.j_after_update[-1] == 0.0


def test_relative_gap_definition():
    y = np.array([[3.0, 4.0]], np.float32)
    c = np.array([[3.0, 3.0], [3.0, 6.0]], np.float32)   # D = 1 and 4
    labels, dist = km.assign(y, c)
    gap = km.relative_gap(dist, labels, y, c)
    # (4 - 1) / (||y||^2 + ||c_0||^2) = 3 / (25 + 18)
    assert gap[0] == pytest.approx(3.0 / 43.0, rel=1e-15)


def test_single_cluster_is_the_exact_mean():
    """C = 1: every token joins the one cluster, no near-tie exists (gap +inf), and
    the centroid is the exactly rounded mean of all tokens (math.fsum per channel)."""
    import math
    rng = np.random.default_rng(4)
    y = (rng.normal(size=(37, 6)) * rng.choice([1.0, 1e3], size=(37, 1))).astype(np.float32)
    tr = km.kmeans(y, 1, 10)
    assert np.all(tr.labels == 0)
    assert all(np.all(np.isinf(g)) for g in tr.gaps_iter)
    mean = np.array([math.fsum(float(v) for v in y[:, k]) / 37 for k in range(6)], np.float64).astype(np.float32)
    assert np.array_equal(tr.centroids[0].view(np.uint32), mean.view(np.uint32))
