"""Rounding helpers of the oracle (test infrastructure only).

* ``bf16_rne``: IEEE float32 -> bfloat16 with round-to-nearest, ties to even.  The
  QVG notes (section "Method / Overall framework") keep centroids in BF16; the
  reading taken for the per-group scale stores it in BF16 too.
* ``group_sums_exact``: per (cluster, channel) sums of float32 values, returned as
  the float64 nearest to the exact real sum.  Used for the k-means centroid update
  (QVG notes, "Semantic-Aware Smoothing": each group's centroid), so that the
  result does not depend on an order of additions.

Pins: ``tests/test_oracle_numerics.py`` checks ``bf16_rne`` against the bit
patterns of hand-worked values and against the fact that every bf16 value is a
fixed point; ``group_sums_exact`` against ``fractions.Fraction`` arithmetic.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_rne(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  Inputs
    must be finite (the oracle refuses NaN/Inf).
    """
    a = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16_rne: non-finite input")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(x) -> np.ndarray:
    """The 16-bit pattern of values that are already bfloat16-exact."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: value is not bfloat16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    """float32 values of 16-bit bfloat16 patterns."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fp32_ulp_lower_bound(v: np.ndarray) -> np.ndarray:
    """A power of two that divides every float32 value ``v`` (v != 0).

    For a normal float32 v = m * 2^e with m in [0.5, 1), the spacing of float32
    numbers at v is 2^(e-24); v is an integer multiple of it.  For subnormals the
    formula gives a smaller power of two, which still divides v.
    """
    _, e = np.frexp(v.astype(np.float64))
    return np.ldexp(1.0, e - 24)


def group_sums_exact(y: np.ndarray, labels: np.ndarray, n_groups: int) -> np.ndarray:
    """Sums of the rows of ``y`` (float32 [N, d]) per label, exactly rounded to fp64.

    Result ``s[j, k]`` is the float64 nearest to the exact sum of ``y[i, k]`` over
    ``labels[i] == j`` (0 for an empty group).

    Fast path with a proof of exactness: every member is an integer multiple of
    ``m`` (the smallest spacing among the members, a power of two), so every
    partial sum is a multiple of ``m`` bounded by ``T = sum |y|``; float64 holds
    every multiple of ``m`` up to ``2**53 * m`` exactly, so if ``T`` is below that
    bound (with a margin for the rounding of ``T`` itself) plain float64
    accumulation in any order is exact.  Otherwise ``math.fsum`` (correctly
    rounded) is used for that (group, channel).
    """
    y = np.asarray(y, dtype=np.float32)
    labels = np.asarray(labels, dtype=np.int64)
    n, d = y.shape
    y64 = y.astype(np.float64)
    sums = np.zeros((n_groups, d), dtype=np.float64)
    abs_sums = np.zeros((n_groups, d), dtype=np.float64)
    np.add.at(sums, labels, y64)
    np.add.at(abs_sums, labels, np.abs(y64))
    nz = y != 0
    spacing = np.where(nz, _fp32_ulp_lower_bound(np.where(nz, y, 1.0)), np.inf)
    min_spacing = np.full((n_groups, d), np.inf)
    np.minimum.at(min_spacing, labels, spacing)
    bound = np.ldexp(min_spacing, 53)
    safe = (abs_sums * (1.0 + 1e-9) < bound) | (abs_sums == 0)
    if not np.all(safe):
        order = np.argsort(labels, kind="stable")
        sorted_labels = labels[order]
        starts = np.searchsorted(sorted_labels, np.arange(n_groups), side="left")
        ends = np.searchsorted(sorted_labels, np.arange(n_groups), side="right")
        for j, k in zip(*np.nonzero(~safe)):
            members = order[starts[j]:ends[j]]
            sums[j, k] = math.fsum(y64[members, k].tolist())
    return sums


def fp32(x) -> np.ndarray:
    """Round to float32 (IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
