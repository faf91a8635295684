"""Pins of oracle.psac: eigenvalues against a 2x2 closed form, the Ky Fan bound by
random frames, projector properties, weights and ranking by hand, and the
closed-form energy of the synthetic query process."""
import math

import numpy as np
import pytest

from oracle import psac
from video_model_kv_amd import synth


def test_two_by_two_closed_form():
    m = np.array([[5.0, 2.0], [2.0, 1.0]])
    u, lam, energy = psac.principal_subspace(m, 1)
    mid, rad = 3.0, math.sqrt(4.0 + 4.0)
    assert lam[0] == pytest.approx(mid + rad, rel=1e-14)
    assert lam[1] == pytest.approx(mid - rad, rel=1e-12)
    assert energy == pytest.approx((mid + rad) / 6.0, rel=1e-14)
    # eigenvector satisfies M u = lambda u
    assert np.allclose(m @ u[:, 0], lam[0] * u[:, 0], atol=1e-13)


@pytest.mark.parametrize("d,r", [(3, 1), (4, 2), (6, 3)])
def test_ky_fan_bound_random_frames(d, r):
    rng = np.random.default_rng(d * 10 + r)
    a = rng.standard_normal((20, d))
    m = a.T @ a
    u, lam, _ = psac.principal_subspace(m, r)
    best = lam[:r].sum()
    assert np.trace(u.T @ m @ u) == pytest.approx(best, rel=1e-12)
    for _ in range(2000):
        v, _ = np.linalg.qr(rng.standard_normal((d, r)))
        assert np.trace(v.T @ m @ v) <= best * (1 + 1e-12)


def test_projector_properties_and_full_rank():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((200, 8))
    u, lam, energy = psac.principal_subspace(psac.query_gram(q), 3)
    p = u @ u.T
    assert np.allclose(p @ p, p, atol=1e-13)
    assert np.allclose(u.T @ u, np.eye(3), atol=1e-13)
    uf, _, ef = psac.principal_subspace(psac.query_gram(q), 8)
    assert ef == pytest.approx(1.0, abs=1e-14)
    assert np.allclose(uf @ uf.T, np.eye(8), atol=1e-12)


def test_weights_and_ranking_by_hand():
    q = np.array([[1.0, 2.0, 0.0, 3.0], [1.0, -2.0, 2.0, 1.0]], np.float32)
    w = psac.qsac_weights(q)
    assert w.tolist() == [1.0, 4.0, 2.0, 5.0]
    assert psac.sensitivity_perm(w, 2).tolist() == [1, 3, 0, 2]
    # ties go to the lower channel index
    assert psac.sensitivity_perm(np.array([2, 1, 2, 2], np.float32), 2).tolist() == [0, 2, 1, 3]


def test_coefficients_round_to_bf16():
    e = np.array([[1.0, 0.0], [0.0, 3.0]], np.float32)
    u = np.array([[1.0], [1.0 / 3.0]])
    c = psac.psac_coefficients(e, u)
    assert c[:, 0].tolist() == [1.0, 1.0]           # 3 * (1/3) in fp64 is 1.0
    assert psac.bf16_rne_f64(1.0 + 2 ** -8) == np.float32(1.0)       # tie -> even
    assert psac.bf16_rne_f64(1.0 + 3 * 2 ** -8) == np.float32(1.0 + 2 ** -6)


def test_synthetic_query_energy_closed_form():
    """Queries q = B a with 8 coordinates of variance 20 and 120 of variance 1:
    the expected top-8 energy is 8*20 / (8*20 + 120) = 0.5714."""
    wl = synth.workload(4)
    hq = synth.history_queries(wl, heads=[0, 7])
    for h in range(2):
        _, _, e = psac.principal_subspace(psac.query_gram(hq[:, h]), 8)
        assert e == pytest.approx(160.0 / 280.0, abs=0.02)


def test_qsac_range_weights_by_hand():
    """Hand-worked chunk: channel ranges 4 - (-2) = 6 and 2 - (-3) = 5, squared
    36 and 25, times the query weights 0.5 and 2."""
    y = np.array([[1.0, -3.0], [4.0, 0.5], [-2.0, 2.0]], np.float32)
    w = np.array([0.5, 2.0], np.float32)
    assert np.array_equal(psac.qsac_range_weights(y, w), np.array([18.0, 50.0], np.float32))


def _ranged_chunk(rng, n, exps):
    """Channel k takes values 2^e_k * (u - 1/4), u on a 1/8 grid in [0, 1] with
    both ends present: range exactly 2^e_k, and max |y| (3/4 of it) differs."""
    u = rng.integers(0, 9, (n, len(exps))) / 8.0
    u[0], u[1] = 0.0, 1.0
    return ((u - 0.25) * (2.0 ** np.asarray(exps, np.float64))).astype(np.float32)


def test_qsac_range_kmeans_equals_plain_kmeans_on_range_scaled_channels():
    """With unit query weights the range factor weighs channel k by rho_k^2, so
    the weighted distance equals the plain distance of the chunk with channel k
    scaled by rho_k.  Ranges that are powers of two make both exact: labels and
    (scaled) centroids must agree bit for bit, through the whole pipeline too."""
    from oracle import kmeans as km
    from oracle import pipeline as pl
    rng = np.random.default_rng(41)
    exps = [-3, 0, 2, 5, 1, -1, 4, 3]
    y = _ranged_chunk(rng, 96, exps)
    rho = (2.0 ** np.asarray(exps, np.float64)).astype(np.float32)
    w_eff = psac.qsac_range_weights(y, np.ones(8, np.float32))
    assert np.array_equal(w_eff, rho * rho)
    a = km.kmeans(y, 6, 10, w_eff)
    b = km.kmeans((y * rho).astype(np.float32), 6, 10, None)
    assert np.array_equal(a.labels, b.labels)
    assert np.array_equal((a.centroids * rho).astype(np.float32), b.centroids)
    res = pl.quantize_problem(y, 6, 2, 4, 1, 10, w=np.ones(8, np.float32), qsac_range=True)
    assert np.array_equal(res.stages[0].labels, b.labels)
    plain = pl.quantize_problem(y, 6, 2, 4, 1, 10, w=np.ones(8, np.float32))
    assert not np.array_equal(plain.stages[0].labels, b.labels), "the factor should change this clustering"
