"""Attention over the dequantized cache, with the PSAC logit correction (oracle;
test infrastructure only).

QVG notes, section "Key designs / Algorithm-system co-design": attention reads the
quantized cache (dequantization x_hat = S q + C_i, "Method / Overall
framework").  QuantWM summary, section "QuantWM", second technique: the stored
projections of the key error on the query principal subspace U are added back
to the logits at inference, i.e. s_ij += (q_i U) . coef_j.

Readings taken: the correction is added before the softmax scale; the scale is
1/sqrt(d) unless given; a causal mask keeps keys j <= i (token order) when the
queries are the cached tokens themselves.  Everything is float64: logits,
softmax and the probability-weighted sum of the float32 V_hat values.

Pins (tests/test_oracle_attention.py): equality with
torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, and a
pure-Python loop on tiny shapes.
"""
from __future__ import annotations

import numpy as np


def logits(q, k_hat, coef=None, u=None, scale=None, causal=False):
    """s [Nq, Nk] for one head (float64); masked entries are -inf."""
    q64 = np.asarray(q, np.float32).astype(np.float64)
    k64 = np.asarray(k_hat, np.float32).astype(np.float64)
    d = q64.shape[1]
    s = q64 @ k64.T
    if coef is not None and u is not None and np.asarray(u).shape[-1] > 0:
        qu = q64 @ np.asarray(u, np.float64)
        s = s + qu @ np.asarray(coef, np.float64).T
    s = s * (1.0 / np.sqrt(d) if not scale else float(scale))
    if causal:
        nq, nk = s.shape
        mask = np.arange(nk)[None, :] > np.arange(nq)[:, None]
        s = np.where(mask, -np.inf, s)
    return s


def attend_head(q, k_hat, v_hat, coef=None, u=None, scale=None, causal=False):
    """O [Nq, d] for one head (float64)."""
    s = logits(q, k_hat, coef, u, scale, causal)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ np.asarray(v_hat, np.float32).astype(np.float64)


def attend(q, k_hat, v_hat, coef=None, u=None, scale=None, causal=False, heads=None):
    """All heads: q [Nq, H, d], k_hat/v_hat [Nk, H, d], coef [Nk, H, r], u [H, d, r].

    Returns {head: O [Nq, d] float64}.
    """
    q = np.asarray(q, np.float32)
    heads = range(q.shape[1]) if heads is None else heads
    out = {}
    for h in heads:
        out[h] = attend_head(q[:, h], k_hat[:, h], v_hat[:, h],
                             None if coef is None else coef[:, h],
                             None if u is None else u[h], scale, causal)
    return out
