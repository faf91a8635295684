"""Lloyd k-means of one chunk's tokens (oracle; test infrastructure only).

Follows the QVG notes, section "Key designs / Semantic-Aware Smoothing": the N
tokens of a chunk are clustered into C groups and each group gets a centroid
(the group mean).  The QuantWM summary, section "QuantWM" (first technique,
QSAC), weights each channel's error by how active the history queries are in
that channel; here that enters as a per-channel weight ``w`` in the distance
(``w = 1`` for plain k-means).

Protocol (fixed, since the pages leave it open):
  * init: centroid j is token j * floor(N / C) (strided rows), in float32;
  * ``iters`` rounds of (assign, update);
  * assign: D[i, j] = sum_k w_k (y_ik - c_jk)^2 in float64 from float32 values,
    label = argmin_j, the lowest j winning exact ties;
  * update: c_j = fp32(fp64(exact sum of members) / n_j), an empty cluster keeps
    its previous centroid;
  * result: labels of the last assign, centroids of the last update.
Near ties: gap_i = (D_(2) - D_(1)) / (||y_i||^2_w + ||c_{l_i}||^2_w) (float64).

Pins (tests/test_oracle_kmeans.py): brute-force argmin over all assignments for
N <= 8; the Lloyd objective never increases; exact recovery of noise-free
prototypes; distances equal a pure-Python double loop.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .numerics import group_sums_exact, fp32


def init_centroids(y: np.ndarray, n_clusters: int) -> np.ndarray:
    """Strided initial centroids: row j * floor(N / C) of the chunk (float32)."""
    y = np.asarray(y, dtype=np.float32)
    n = y.shape[0]
    if n < n_clusters:
        raise ValueError("k-means needs at least as many tokens as clusters")
    step = n // n_clusters
    return y[np.arange(n_clusters) * step].copy()


def sq_distances(y: np.ndarray, c: np.ndarray, w: np.ndarray | None = None) -> np.ndarray:
    """D[i, j] = sum_k w_k (y_ik - c_jk)^2, in float64 (direct form, channel by channel)."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    d = y64.shape[1]
    w64 = np.ones(d) if w is None else np.asarray(w, dtype=np.float32).astype(np.float64)
    dist = np.zeros((y64.shape[0], c64.shape[0]), dtype=np.float64)
    for k in range(d):
        diff = y64[:, k:k + 1] - c64[None, :, k]
        dist += w64[k] * (diff * diff)
    return dist


def assign(y, c, w=None):
    """Labels (int64) = argmin over centroids, lowest index on exact ties; and D."""
    dist = sq_distances(y, c, w)
    labels = np.argmin(dist, axis=1)  # numpy returns the first minimum
    return labels, dist


def update(y, labels, c_old):
    """New centroids: exact group mean rounded to float32; empty cluster keeps c_old."""
    y = np.asarray(y, dtype=np.float32)
    n_clusters = c_old.shape[0]
    counts = np.bincount(labels, minlength=n_clusters)
    sums = group_sums_exact(y, labels, n_clusters)
    c_new = np.asarray(c_old, dtype=np.float32).copy()
    nonempty = counts > 0
    c_new[nonempty] = fp32(sums[nonempty] / counts[nonempty, None].astype(np.float64))
    return c_new, counts


def objective(dist: np.ndarray, labels: np.ndarray) -> float:
    """Lloyd objective J = sum_i D[i, label_i] (float64)."""
    return float(dist[np.arange(dist.shape[0]), labels].sum())


def relative_gap(dist: np.ndarray, labels: np.ndarray, y, c, w=None) -> np.ndarray:
    """(second-smallest D - smallest D) / (||y_i||^2_w + ||c_label||^2_w), float64.
    With a single centroid there is no second candidate: the gap is +inf."""
    if dist.shape[1] < 2:
        return np.full(dist.shape[0], np.inf)
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    w64 = np.ones(y64.shape[1]) if w is None else np.asarray(w, np.float32).astype(np.float64)
    part = np.partition(dist, 1, axis=1)
    num = part[:, 1] - part[:, 0]
    den = (y64 * y64 * w64).sum(1) + (c64[labels] ** 2 * w64).sum(1)
    return num / np.where(den > 0, den, 1.0)


@dataclass
class KMeansTrace:
    """Everything one k-means run produced, kept for lock-step comparisons."""
    labels: np.ndarray                      # int64 [N], from the last assign
    centroids: np.ndarray                   # float32 [C, d], from the last update
    counts: np.ndarray                      # int64 [C], from the last update
    centroids_in: list = field(default_factory=list)   # float32 [C, d] before each assign
    labels_iter: list = field(default_factory=list)    # labels of each assign
    gaps_iter: list = field(default_factory=list)      # relative gap of each assign
    j_after_assign: list = field(default_factory=list)
    j_after_update: list = field(default_factory=list)


def kmeans(y, n_clusters: int, iters: int = 10, w=None, init=None,
           track_objective: bool = True) -> KMeansTrace:
    """Run the fixed protocol; ``init`` overrides the strided initial centroids.

    With ``track_objective`` the Lloyd objective is recorded after every assign
    and every update (the latter costs one more distance evaluation at the end).
    """
    y = np.asarray(y, dtype=np.float32)
    c = init_centroids(y, n_clusters) if init is None else np.asarray(init, np.float32).copy()
    tr = KMeansTrace(labels=None, centroids=None, counts=None)
    labels = None
    for _ in range(iters):
        tr.centroids_in.append(c.copy())
        new_labels, dist = assign(y, c, w)
        if labels is not None and track_objective:
            tr.j_after_update.append(objective(dist, labels))
        labels = new_labels
        tr.labels_iter.append(labels)
        tr.gaps_iter.append(relative_gap(dist, labels, y, c, w))
        if track_objective:
            tr.j_after_assign.append(objective(dist, labels))
        c, counts = update(y, labels, c)
        tr.counts = counts
    if track_objective and labels is not None:
        tr.j_after_update.append(objective(sq_distances(y, c, w), labels))
    tr.labels = labels
    tr.centroids = c
    return tr
