"""GPU parity of the autoregressive chunk loop: each step attends the new chunk's
queries over the packed cache followed by the chunk's own bf16 keys and values
(frame-block causal), then quantizes the chunk and appends it to the cache.
The oracle quantizes the checked heads itself and attends with
oracle.attention.attend_fresh.  Bars: logits within 1e-3 and outputs within
5e-3 relative L2; the appended chunks bit for bit."""
import numpy as np
import pytest

import video_model_kv_amd as qk
from video_model_kv_amd import synth
from oracle import attention as oa
from oracle import psac as ops

import gpu_helpers as G

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-3
OUT_TOL = 5e-3


def _rollout(name, wl, heads, n_steps):
    t = G.torch()
    H, F = wl.n_heads, wl.tokens_per_frame
    kcfg, vcfg = G.config_of(wl, "K"), G.config_of(wl, "V")
    w = u = perm = None
    if wl.qsac or wl.psac_rank or wl.n_int4:
        hist = synth.history_queries(wl)
        wl_ = [ops.qsac_weights(hist[:, h]) for h in range(H)]
        w = np.stack(wl_) if wl.qsac else None
        u = (np.stack([ops.principal_subspace(ops.query_gram(hist[:, h]), wl.psac_rank)[0] for h in range(H)])
             .astype(np.float32) if wl.psac_rank else None)
        perm = np.stack([ops.sensitivity_perm(x, wl.n_int4) for x in wl_]) if wl.n_int4 else None
    wd = None if w is None else G.to_dev(w)
    ud = None if u is None else G.to_dev(u)
    pd = None if perm is None else t.from_numpy(perm.astype(np.uint8)).to(G.dev())
    n_max = wl.chunk_tokens
    ws = G.workspace(kcfg, n_max, n_max, n_steps)
    kch, vch, ntok = [], [], []
    k_hat = {h: [] for h in heads}
    v_hat = {h: [] for h in heads}
    coef = {h: [] for h in heads}
    for c in range(n_steps):
        a, b = wl.chunk_range(c)
        k = synth.kv_tokens(wl, "K", a, b)
        v = synth.kv_tokens(wl, "V", a, b)
        q = synth.chunk_queries(wl, c)
        kd, vd, qd = G.to_dev(k, "bf16"), G.to_dev(v, "bf16"), G.to_dev(q, "bf16")
        nf = b - a
        nk = sum(ntok) + nf
        out = t.empty((nf, H, 128), dtype=t.float32, device=G.dev())
        logits = t.empty((H, nf, nk), dtype=t.float32, device=G.dev())
        G.log(f"ar {name} step {c}: cache {len(kch)} chunks ({sum(ntok)} keys), fresh {nf}, frame {F}")
        qk.qkv_attend_fresh(kcfg, vcfg, qd, kch, vch, ntok, kd, vd, F, out, ws, U=ud, logits=logits)
        o = out.cpu().numpy()
        lg = logits.cpu().numpy()
        for h in heads:
            kc = np.concatenate(k_hat[h]) if k_hat[h] else np.zeros((0, 128), np.float32)
            vc = np.concatenate(v_hat[h]) if v_hat[h] else np.zeros((0, 128), np.float32)
            cf = np.concatenate(coef[h]) if (u is not None and coef[h]) else None
            uh = None if u is None else u[h].astype(np.float64)
            if cf is None and uh is not None:
                cf = np.zeros((0, uh.shape[1]))
            ref = oa.attend_fresh(q[:, h], kc, vc, k[:, h], v[:, h], F, cf, uh)
            s_ref = oa.logits_fresh(q[:, h], kc, k[:, h], F, cf, uh)
            fin = np.isfinite(s_ref)
            assert np.array_equal(fin, np.isfinite(lg[h])), f"ar {name} step {c} h{h}: mask differs"
            e_log = G.rel_l2(lg[h][fin], s_ref[fin])
            e_out = G.rel_l2(o[:, h], ref)
            G.log(f"ar {name} step {c} h{h}: rel-L2 logits {e_log:.3g}, out {e_out:.3g}")
            assert e_log <= LOGIT_TOL and e_out <= OUT_TOL, f"ar {name} step {c} h{h}: {e_log} {e_out}"
        # append: the chunk's write path, checked bit for bit on the sampled heads
        kch.append(G.quantize(kcfg, kd, w=wd, perm=pd, u=ud))
        vch.append(G.quantize(vcfg, vd))
        ntok.append(nf)
        jobs = []
        for h in heads:
            jobs.append((k[:, h], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                                       iters=wl.kmeans_iters, w=None if w is None else w[h],
                                       n_int4=kcfg.n_int4_channels, perm=None if perm is None else perm[h],
                                       u=None if u is None else u[h].astype(np.float64))))
            jobs.append((v[:, h], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                                       iters=wl.kmeans_iters)))
        res = G.oracle_problems(jobs)
        G.compare_chunk(f"ar {name} chunk {c} K", wl, "K", k, kch[-1], kcfg, {h: res[2 * i] for i, h in enumerate(heads)},
                        heads)
        G.compare_chunk(f"ar {name} chunk {c} V", wl, "V", v, vch[-1], vcfg,
                        {h: res[2 * i + 1] for i, h in enumerate(heads)}, heads)
        for i, h in enumerate(heads):
            k_hat[h].append(res[2 * i].x_hat)
            v_hat[h].append(res[2 * i + 1].x_hat)
            if u is not None:
                coef[h].append(res[2 * i].coef)


def _small(cid, **over):
    return synth.workload(cid, n_heads=2, n_clusters=32, frames=6, chunk_frames=2, tokens_per_frame=260, **over)


def test_ar_rollout_int2():
    _rollout("int2", _small(2), [0, 1], 3)


def test_ar_rollout_mixed_keys():
    """Mixed INT4/INT2 keys (the mix4 attention path) with fresh chunks."""
    _rollout("mixed", _small(5), [1], 3)


def test_ar_rollout_psac():
    """QSAC-weighted k-means and PSAC on the cached keys; the fresh keys carry no correction."""
    _rollout("psac", _small(4), [0], 3)


def test_ar_rollout_two_stages():
    """Two progressive stages (the generic decode) with fresh chunks."""
    _rollout("progressive", _small(3, n_stages=2), [1], 3)


def test_ar_first_step_and_ragged_frames():
    """The first step (no cache) and a frame size that does not divide the 64-key tiles."""
    wl = synth.workload(2, n_heads=2, n_clusters=16, frames=4, chunk_frames=2, tokens_per_frame=97)
    _rollout("ragged", wl, [0], 2)
