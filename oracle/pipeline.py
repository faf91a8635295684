"""One KV chunk through the whole write path, and back (oracle; test
infrastructure only).

Per (head, tensor) problem, following the QVG notes, section "Method / Overall
framework" and the two designs under "Key designs":
  1. k-means of the chunk's N tokens into C groups (oracle.kmeans);
  2. centroids stored in bf16, C_bf16 = bf16(c);
  3. residual r = fp32(y - C_bf16[label]) (taken against the stored centroid, so
     that the dequantized value rebuilds what was quantized);
  4. per-group symmetric quantization of r (oracle.quant);
  5. progressive residual stages ("Progressive Residual Quantization"): the
     next stage's input is Y_{l+1} = fp32(Y_l - Yhat_l) and each stage runs its
     own k-means; X_hat = Yhat_1 + Yhat_2 + ... summed in float32 in stage order;
  1a. with ``qsac_range`` the k-means weights of each stage are QSAC's weights
     times the squared range of each channel of that stage's input
     (oracle.psac.qsac_range_weights; QuantWM summary, first technique);
  6. PSAC encode (QuantWM summary, "QuantWM", second technique), keys only:
     e = fp32(K - K_hat) after all stages, coef = bf16(U^T e).
A test-only switch ``rtn`` replaces steps 1-2 by zero centroids (plain
round-to-nearest per-group quantization, the "RTN" row of the QVG notes' main
table and the "no clustering" ablation).

Parity status: every step is pinned by the tests named in the step's module;
the whole chain is additionally pinned by the reconstruction identity and by
the RTN special case (tests/test_oracle_pipeline.py).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import kmeans as km
from .numerics import bf16_rne
from .psac import psac_coefficients, qsac_range_weights
from .quant import channel_layout, quantize_groups, dequantize


@dataclass
class StageResult:
    labels: np.ndarray        # int64 [N]
    centroids: np.ndarray     # float32 [C, d] (k-means output)
    centroids_bf16: np.ndarray  # float32 values, bf16-exact [C, d]
    q: np.ndarray             # int8 [N, d]
    scales: np.ndarray        # float32, bf16-exact [N, groups]
    y_in: np.ndarray          # float32 [N, d] this stage's input
    y_hat: np.ndarray         # float32 [N, d]
    trace: km.KMeansTrace | None = None


@dataclass
class ProblemResult:
    stages: list = field(default_factory=list)
    x_hat: np.ndarray | None = None     # float32 [N, d]
    coef: np.ndarray | None = None      # float32, bf16-exact [N, r]
    layout: object = None


def quantize_problem(x, n_clusters: int, bits: int, group: int, n_stages: int = 1,
                     iters: int = 10, w=None, n_int4: int = 0, perm=None, u=None,
                     rtn: bool = False, track_objective: bool = False,
                     qsac_range: bool = False) -> ProblemResult:
    """Quantize one (head, tensor) problem: x is float32 [N, d] (bf16 values allowed).
    ``qsac_range`` (needs ``w``): each stage's k-means weights get the stage
    input's squared channel ranges as a second factor."""
    if qsac_range and w is None:
        raise ValueError("qsac_range needs the QSAC weights w")
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    n, d = x.shape
    layout = channel_layout(d, bits, group, n_int4, perm)
    res = ProblemResult(layout=layout)
    y = x
    x_hat = None
    for _ in range(n_stages):
        if rtn:
            labels = np.zeros(n, np.int64)
            cent = np.zeros((n_clusters, d), np.float32)
            trace = None
        else:
            w_stage = qsac_range_weights(y, w) if qsac_range else w
            trace = km.kmeans(y, n_clusters, iters, w_stage, track_objective=track_objective)
            labels, cent = trace.labels, trace.centroids
        c_bf = bf16_rne(cent)
        rows = c_bf[labels]
        r = (y - rows).astype(np.float32)
        q, scales = quantize_groups(r, layout)
        y_hat = dequantize(q, scales, rows, layout)
        res.stages.append(StageResult(labels, cent, c_bf, q, scales, y, y_hat, trace))
        x_hat = y_hat if x_hat is None else (x_hat + y_hat).astype(np.float32)
        y = (y - y_hat).astype(np.float32)
    res.x_hat = x_hat
    if u is not None and np.asarray(u).shape[1] > 0:
        e = (x - x_hat).astype(np.float32)
        res.coef = psac_coefficients(e, u)
    return res


def quantize_chunk(x, n_clusters: int, bits: int, group: int, n_stages: int = 1,
                   iters: int = 10, w=None, n_int4: int = 0, perm=None, u=None,
                   rtn: bool = False, heads=None, qsac_range: bool = False) -> dict:
    """All heads (or the listed ``heads``) of one chunk x [N, H, d].

    ``w`` [H, d], ``perm`` [H, d] and ``u`` [H, d, r] are per-head side inputs
    (None when off).  Returns {head: ProblemResult}.
    """
    x = np.asarray(x, dtype=np.float32)
    heads = range(x.shape[1]) if heads is None else heads
    out = {}
    for h in heads:
        out[h] = quantize_problem(
            x[:, h, :], n_clusters, bits, group, n_stages, iters,
            None if w is None else w[h], n_int4,
            None if perm is None else perm[h], None if u is None else u[h], rtn, qsac_range=qsac_range)
    return out


def dequantize_stages(stages, layout) -> np.ndarray:
    """X_hat from the stored fields of each stage (codes, scales, labels, bf16
    centroids): the float32 sum over stages of fp32(S * q + C_bf16[label])."""
    x_hat = None
    for st in stages:
        y_hat = dequantize(st.q, st.scales, st.centroids_bf16[st.labels], layout)
        x_hat = y_hat if x_hat is None else (x_hat + y_hat).astype(np.float32)
    return x_hat
