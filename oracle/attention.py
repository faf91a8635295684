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

Autoregressive chunk step (QVG notes, "Research background": chunk-by-chunk
generation with causal attention over a resident KV cache; "Method / Overall
framework": the cache is written chunk by chunk; 2-bit trap explainer, opening:
every new frame attends to all cached frames).  Readings taken: the queries of
a step are the new chunk's own tokens; they see every cached (quantized) key and
the new chunk's own keys, unquantized, of frames up to their own frame
(frame-block causal); the PSAC term applies to cached keys only (fresh keys
carry no quantization error).

Pins (tests/test_oracle_attention.py): equality with
torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, and a
pure-Python loop on tiny shapes; for the chunk step, the one-frame and
one-token special cases (full and token-causal attention) and a Python loop
over the visibility rule.
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


def fresh_visible(nq: int, n_cache: int, n_fresh: int, frame_tokens: int, q_index=None) -> np.ndarray:
    """Visibility [nq, n_cache + n_fresh] of one autoregressive chunk step: query i
    (token q_index[i] of the new chunk; default i) sees every cached key and fresh
    key j iff j // frame_tokens <= q_index[i] // frame_tokens."""
    qi = np.arange(nq) if q_index is None else np.asarray(q_index)
    qf = qi // frame_tokens
    kf = np.arange(n_fresh) // frame_tokens
    fresh = kf[None, :] <= qf[:, None]
    return np.concatenate([np.ones((nq, n_cache), bool), fresh], axis=1)


def logits_fresh(q, k_hat_cache, k_fresh, frame_tokens: int, coef=None, u=None, scale=None, q_index=None):
    """s [Nq, Nc + Nf] of a chunk step (float64), -inf where not visible; the PSAC
    term (coef [Nc, r]) is added for the cached keys only.  q_index: the chunk
    token of each query row (a subset of the chunk's queries), default 0..Nq-1."""
    k_all = np.concatenate([np.asarray(k_hat_cache, np.float32).reshape(-1, np.asarray(k_fresh).shape[1]),
                            np.asarray(k_fresh, np.float32)])
    nc = k_all.shape[0] - np.asarray(k_fresh).shape[0]
    c_all = None
    if coef is not None and u is not None and np.asarray(u).shape[-1] > 0:
        r = np.asarray(u).shape[-1]
        c_all = np.concatenate([np.asarray(coef, np.float64).reshape(nc, r), np.zeros((k_all.shape[0] - nc, r))])
    s = logits(q, k_all, c_all, u if c_all is not None else None, scale)
    vis = fresh_visible(s.shape[0], nc, k_all.shape[0] - nc, frame_tokens, q_index)
    return np.where(vis, s, -np.inf)


def attend_fresh(q, k_hat_cache, v_hat_cache, k_fresh, v_fresh, frame_tokens: int, coef=None, u=None, scale=None,
                 q_index=None):
    """O [Nq, d] of one autoregressive chunk step for one head (float64)."""
    s = logits_fresh(q, k_hat_cache, k_fresh, frame_tokens, coef, u, scale, q_index)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    d = np.asarray(v_fresh).shape[1]
    v_all = np.concatenate([np.asarray(v_hat_cache, np.float32).reshape(-1, d), np.asarray(v_fresh, np.float32)])
    return p @ v_all.astype(np.float64)
