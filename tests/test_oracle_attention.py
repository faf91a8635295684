"""Pins of oracle.attention: torch scaled-dot-product attention in float64 on the
CPU, a pure-Python loop on tiny shapes, and PSAC full-rank exactness."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, psac


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    rng = np.random.default_rng(0)
    q = rng.standard_normal((40, 3, 32)).astype(np.float32)
    k = (rng.standard_normal((40, 3, 32)) * 3).astype(np.float32)
    v = (rng.standard_normal((40, 3, 32)) * 10).astype(np.float32)
    out = attention.attend(q, k, v, causal=causal)
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    for h in range(3):
        assert np.allclose(out[h], ref[h].numpy(), rtol=1e-12, atol=1e-12)


def test_python_loop_tiny_with_psac():
    rng = np.random.default_rng(1)
    nq, nk, d, r = 5, 7, 4, 2
    q = rng.standard_normal((nq, d)).astype(np.float32)
    k = rng.standard_normal((nk, d)).astype(np.float32)
    v = rng.standard_normal((nk, d)).astype(np.float32)
    u = np.linalg.qr(rng.standard_normal((d, r)))[0]
    coef = rng.standard_normal((nk, r)).astype(np.float32)
    o = attention.attend_head(q, k, v, coef, u, scale=0.3)
    for i in range(nq):
        s = []
        for j in range(nk):
            dot = sum(float(q[i, a]) * float(k[j, a]) for a in range(d))
            qu = [sum(float(q[i, a]) * u[a, b] for a in range(d)) for b in range(r)]
            dot += sum(qu[b] * float(coef[j, b]) for b in range(r))
            s.append(0.3 * dot)
        m = max(s)
        p = [math.exp(x - m) for x in s]
        z = sum(p)
        for a in range(d):
            ref = sum(p[j] / z * float(v[j, a]) for j in range(nk))
            assert o[i, a] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_psac_full_rank_recovers_exact_logits():
    rng = np.random.default_rng(2)
    d = 16
    qh = rng.standard_normal((300, d))
    u, _, _ = psac.principal_subspace(psac.query_gram(qh), d)
    k = (rng.standard_normal((50, d)) * 5).astype(np.float32)
    k_hat = np.round(k).astype(np.float32)           # any approximation
    e = (k.astype(np.float64) - k_hat.astype(np.float64))
    coef = e @ u                                      # unrounded coefficients
    q = rng.standard_normal((9, d)).astype(np.float32)
    s_corr = attention.logits(q, k_hat, coef, u)
    s_true = attention.logits(q, k)
    assert np.allclose(s_corr, s_true, rtol=0, atol=1e-12)
    # rank 0: no correction
    assert np.array_equal(attention.logits(q, k_hat, coef[:, :0], u[:, :0]), attention.logits(q, k_hat))


def test_chunk_step_special_cases():
    """One frame per chunk: the fresh keys are all visible (full attention over
    cache + chunk); one token per frame and no cache: token-causal attention."""
    rng = np.random.default_rng(3)
    d, nc, nf = 16, 11, 9
    q = rng.standard_normal((nf, d)).astype(np.float32)
    kc, vc = rng.standard_normal((nc, d)).astype(np.float32), rng.standard_normal((nc, d)).astype(np.float32)
    kf, vf = rng.standard_normal((nf, d)).astype(np.float32), rng.standard_normal((nf, d)).astype(np.float32)
    full = attention.attend_head(q, np.concatenate([kc, kf]), np.concatenate([vc, vf]))
    assert np.allclose(attention.attend_fresh(q, kc, vc, kf, vf, frame_tokens=nf), full, rtol=1e-13, atol=1e-13)
    empty = np.zeros((0, d), np.float32)
    causal = attention.attend_head(q, kf, vf, causal=True)
    assert np.allclose(attention.attend_fresh(q, empty, empty, kf, vf, frame_tokens=1), causal, rtol=1e-13, atol=1e-13)


def test_chunk_step_python_loop_with_psac():
    """Visibility by a Python loop: cached keys always, fresh key j iff its frame
    j // F is at most the query's frame i // F; the PSAC term on cached keys only."""
    rng = np.random.default_rng(4)
    d, r, nc, nf, F = 4, 2, 3, 6, 2
    q = rng.standard_normal((nf, d)).astype(np.float32)
    kc, vc = rng.standard_normal((nc, d)).astype(np.float32), rng.standard_normal((nc, d)).astype(np.float32)
    kf, vf = rng.standard_normal((nf, d)).astype(np.float32), rng.standard_normal((nf, d)).astype(np.float32)
    u = np.linalg.qr(rng.standard_normal((d, r)))[0]
    coef = rng.standard_normal((nc, r)).astype(np.float32)
    o = attention.attend_fresh(q, kc, vc, kf, vf, F, coef, u, scale=0.5)
    keys = [(kc[j], vc[j], coef[j], None) for j in range(nc)] + [(kf[j], vf[j], None, j) for j in range(nf)]
    for i in range(nf):
        s, vals = [], []
        for k, v, c, jf in keys:
            if jf is not None and jf // F > i // F:
                continue
            dot = sum(float(q[i, a]) * float(k[a]) for a in range(d))
            if c is not None:
                qu = [sum(float(q[i, a]) * u[a, b] for a in range(d)) for b in range(r)]
                dot += sum(qu[b] * float(c[b]) for b in range(r))
            s.append(0.5 * dot)
            vals.append(v)
        m = max(s)
        p = [math.exp(x - m) for x in s]
        z = sum(p)
        for a in range(d):
            ref = sum(p[j] / z * float(vals[j][a]) for j in range(len(s)))
            assert o[i, a] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_chunk_step_query_subset():
    """Rows for a subset of the chunk's queries (q_index) equal those rows of the
    whole step."""
    rng = np.random.default_rng(5)
    d, nc, nf, F = 8, 5, 12, 4
    q = rng.standard_normal((nf, d)).astype(np.float32)
    kc, vc = rng.standard_normal((nc, d)).astype(np.float32), rng.standard_normal((nc, d)).astype(np.float32)
    kf, vf = rng.standard_normal((nf, d)).astype(np.float32), rng.standard_normal((nf, d)).astype(np.float32)
    full = attention.attend_fresh(q, kc, vc, kf, vf, F)
    idx = np.array([0, 3, 4, 11])
    sub = attention.attend_fresh(q[idx], kc, vc, kf, vf, F, q_index=idx)
    assert np.array_equal(sub, full[idx])


def test_chunk_step_empty_cache_with_psac():
    """First step of a rollout: no cached keys, so the PSAC term (which belongs to
    cached keys only) has nothing to act on; one token per frame makes the step
    token-causal attention over the fresh keys."""
    rng = np.random.default_rng(6)
    d, r, nf = 8, 3, 7
    q = rng.standard_normal((nf, d)).astype(np.float32)
    kf, vf = rng.standard_normal((nf, d)).astype(np.float32), rng.standard_normal((nf, d)).astype(np.float32)
    u = np.linalg.qr(rng.standard_normal((d, r)))[0]
    empty = np.zeros((0, d), np.float32)
    o = attention.attend_fresh(q, empty, empty, kf, vf, 1, np.zeros((0, r), np.float32), u)
    causal = attention.attend_head(q, kf, vf, causal=True)
    assert np.allclose(o, causal, rtol=1e-13, atol=1e-13)
