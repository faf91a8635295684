"""History-query statistics: QSAC channel weights, PSAC principal subspace and the
channel-sensitivity ranking (oracle; test infrastructure only).

* QSAC weights (QuantWM summary, section "QuantWM", first technique): how active
  the history queries are in each channel, read as the mean square
  w_k = mean_n q_nk^2 (float64, rounded once to float32).
* PSAC subspace (same section, second technique): eigendecompose the history
  queries' second-moment matrix M = sum_n q_n q_n^T, keep the r eigenvectors of
  the largest eigenvalues as U (d x r); energy = sum of those r eigenvalues over
  the trace.  The key residual error e is projected onto U and the r
  coefficients are stored (bf16 here; the page says only that they are
  stored quantized); attention adds (q U) . coef back to the logit.
* QSAC's second factor (same section, first technique: besides the channels'
  query activity, the clustering weighs the dynamic range of the residual being
  quantized, and combines both).  Reading: the weight of channel k for the
  k-means of one stage is w_k * rho_k^2, rho_k the range (max - min over the
  chunk's tokens) of channel k of that stage's input -- the data at stage 1,
  the previous stages' residual after -- since a channel's range sets its
  group's quantization step.  In float32: rho = fl(max - min),
  w_eff = fl(w * fl(rho * rho)).
* Sensitivity ranking for mixed precision (2-bit trap explainer, section five;
  practitioner blog, section 3.2): the channels with the largest query energy
  w_k get 4 bits; ties go to the lower channel index.

Pins (tests/test_oracle_psac.py): eigenvalues against a 2x2 closed form and
numpy.linalg.eigh, the Ky Fan bound by random r-frames for d <= 6, projector
idempotence, full-rank exactness of the corrected logits; the range weights by
a hand-worked chunk, and weighted k-means with them equal to plain k-means on
the chunk with each channel scaled by its range (powers of two, exact).
"""
from __future__ import annotations

import math

import numpy as np


def query_gram(q: np.ndarray) -> np.ndarray:
    """M = sum_n q_n q_n^T in float64 (q: [n, d])."""
    q64 = np.asarray(q, dtype=np.float32).astype(np.float64)
    return q64.T @ q64


def qsac_weights(q: np.ndarray) -> np.ndarray:
    """w_k = fp32(fp64(exact sum_n q_nk^2) / n)."""
    q64 = np.asarray(q, dtype=np.float32).astype(np.float64)
    n, d = q64.shape
    sums = np.array([math.fsum((q64[:, k] * q64[:, k]).tolist()) for k in range(d)])
    return (sums / float(n)).astype(np.float32)


def qsac_range_weights(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """QSAC weights with the residual-range factor for one stage's input y
    [N, d]: fl32(w_k * fl32(rho_k^2)), rho_k = fl32(max_i y_ik - min_i y_ik)."""
    y = np.asarray(y, dtype=np.float32)
    rho = (y.max(axis=0) - y.min(axis=0)).astype(np.float32)
    return (np.asarray(w, np.float32) * (rho * rho).astype(np.float32)).astype(np.float32)


def principal_subspace(m: np.ndarray, rank: int):
    """Top-``rank`` eigenvectors U (float64 [d, rank], descending eigenvalue),
    all eigenvalues (descending) and the energy fraction they capture."""
    lam, vec = np.linalg.eigh(np.asarray(m, np.float64))
    order = np.argsort(lam)[::-1]
    lam, vec = lam[order], vec[:, order]
    total = lam.sum()
    energy = float(lam[:rank].sum() / total) if total > 0 else 0.0
    return vec[:, :rank].copy(), lam, energy


def sensitivity_perm(w: np.ndarray, n_int4: int) -> np.ndarray:
    """Channel order: the n_int4 largest-w channels (ascending index), then the rest
    (ascending index).  Ranking: larger w first, equal w -> lower index first."""
    w = np.asarray(w, dtype=np.float32)
    d = w.shape[0]
    rank = sorted(range(d), key=lambda k: (-float(w[k]), k))
    top = sorted(rank[:n_int4])
    rest = sorted(rank[n_int4:])
    return np.array(top + rest, dtype=np.int64)


def bf16_rne_f64(x) -> np.ndarray:
    """Round float64 values straight to the nearest bfloat16 (ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, |m| in [0.5, 1)
    r = np.rint(np.ldexp(m, 8))        # 8 significant bits, ties to even
    return np.ldexp(r, e - 8).astype(np.float32)


def psac_coefficients(e: np.ndarray, u: np.ndarray) -> np.ndarray:
    """coef = bf16(U^T e) per token, from float64 dot products (float32 values)."""
    e64 = np.asarray(e, dtype=np.float32).astype(np.float64)
    return bf16_rne_f64(e64 @ np.asarray(u, np.float64))
