"""GPU parity of the attention over the packed cache against the oracle
(attention in float64 over the oracle's own dequantized cache, with the PSAC
term).  Bar: logits within 1e-3 and outputs within 5e-3 relative L2."""
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


def _run(name, wl, chunk_bounds, nq, heads_checked, causal=False, logit_queries=64, q_scale=1.0,
         kv_scale=(1.0, 1.0), softmax_scale=0.0):
    t = G.torch()
    H = wl.n_heads
    kcfg, vcfg = G.config_of(wl, "K"), G.config_of(wl, "V")
    w = u = perm = None
    if wl.qsac or wl.psac_rank or wl.n_int4:
        hist = synth.history_queries(wl)
        wlist = [ops.qsac_weights(hist[:, h]) for h in range(H)]
        if wl.qsac:
            w = np.stack(wlist)
        if wl.psac_rank:
            u = np.stack([ops.principal_subspace(ops.query_gram(hist[:, h]), wl.psac_rank)[0]
                          for h in range(H)]).astype(np.float32)
        if wl.n_int4:
            perm = np.stack([ops.sensitivity_perm(x, wl.n_int4) for x in wlist])
    wd = None if w is None else G.to_dev(w)
    ud = None if u is None else G.to_dev(u)
    pd = None if perm is None else t.from_numpy(perm.astype(np.uint8)).to(G.dev())
    kch, vch, ntok, xk, xv = [], [], [], [], []
    maxn = max(b - a for a, b in chunk_bounds)
    ws = G.workspace(kcfg, maxn, nq, len(chunk_bounds))
    wsv = G.workspace(vcfg, maxn)
    for a, b in chunk_bounds:
        k = synth.kv_tokens(wl, "K", a, b) * np.float32(kv_scale[0])      # powers of two: still bf16-exact
        v = synth.kv_tokens(wl, "V", a, b) * np.float32(kv_scale[1])
        xk.append(k)
        xv.append(v)
        kch.append(G.quantize(kcfg, G.to_dev(k, wl.dtype), w=wd, perm=pd, u=ud, ws=ws))
        vch.append(G.quantize(vcfg, G.to_dev(v, wl.dtype), ws=wsv))
        ntok.append(b - a)
    q = synth.queries(wl, n=nq) * np.float32(q_scale)     # a power of two keeps bf16 queries exact
    qd = G.to_dev(q, wl.dtype)
    out = t.empty((nq, H, 128), dtype=t.float32, device=G.dev())
    G.log(f"attend {name}: H={H} chunks={len(ntok)} Nk={sum(ntok)} Nq={nq} causal={causal} psac={kcfg.psac_rank}")
    qk.qkv_attend(kcfg, vcfg, qd, kch, vch, ntok, out, ws, U=ud, causal=causal, softmax_scale=softmax_scale)
    nk = sum(ntok)
    nlq = min(logit_queries, nq)
    logits = t.empty((H, nq, nk), dtype=t.float32, device=G.dev())
    out2 = t.empty_like(out)
    qk.qkv_attend(kcfg, vcfg, qd, kch, vch, ntok, out2, ws, U=ud, causal=causal, softmax_scale=softmax_scale,
                  logits=logits)
    o = out.cpu().numpy()
    assert np.array_equal(o, out2.cpu().numpy()), "the logits debug path changed the output"
    # oracle: quantize the checked heads itself, then attend in float64
    jobs = []
    for ci in range(len(chunk_bounds)):
        for h in heads_checked:
            for tensor, xs, cfg in (("K", xk, kcfg), ("V", xv, vcfg)):
                jobs.append((xs[ci][:, h], dict(
                    n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                    iters=wl.kmeans_iters, w=None if (w is None or tensor == "V") else w[h],
                    n_int4=cfg.n_int4_channels, perm=None if (perm is None or tensor == "V") else perm[h],
                    u=None if (u is None or tensor == "V") else u[h].astype(np.float64))))
    res = G.oracle_problems(jobs)
    # the packed caches themselves, bit for bit (labels, centroids, codes, scales, PSAC coefficients)
    near = 0
    for ci in range(len(chunk_bounds)):
        for ti, (tensor, chunks, xs, cfg) in enumerate((("K", kch, xk, kcfg), ("V", vch, xv, vcfg))):
            by_head = {h: res[(ci * len(heads_checked) + hi) * 2 + ti] for hi, h in enumerate(heads_checked)}
            near += G.compare_chunk(f"{name} chunk {ci} {tensor}", wl, tensor, xs[ci], chunks[ci], cfg, by_head,
                                    heads_checked)
    G.log(f"attend {name}: packed K/V bit-exact on heads {list(heads_checked)} of {len(chunk_bounds)} chunks "
          f"(near-ties in the oracle's traces: {near})")
    lg = logits[:, :nlq].cpu().numpy()
    for hi, h in enumerate(heads_checked):
        k_hat = np.concatenate([res[(ci * len(heads_checked) + hi) * 2].x_hat for ci in range(len(chunk_bounds))])
        v_hat = np.concatenate([res[(ci * len(heads_checked) + hi) * 2 + 1].x_hat for ci in range(len(chunk_bounds))])
        coef = None
        if u is not None:
            coef = np.concatenate([res[(ci * len(heads_checked) + hi) * 2].coef for ci in range(len(chunk_bounds))])
        sc = softmax_scale or None
        ref = oa.attend_head(q[:, h], k_hat, v_hat, coef, None if u is None else u[h].astype(np.float64),
                             scale=sc, causal=causal)
        e_out = G.rel_l2(o[:, h], ref)
        s_ref = oa.logits(q[:nlq, h], k_hat, coef, None if u is None else u[h].astype(np.float64), scale=sc,
                          causal=causal)
        fin = np.isfinite(s_ref)
        assert np.array_equal(fin, np.isfinite(lg[h])), f"{name} h{h}: mask differs"
        e_log = G.rel_l2(lg[h][fin], s_ref[fin])
        # the unquantized cache, for the quality diagnostic only
        kx = np.concatenate([x[:, h] for x in xk])
        vx = np.concatenate([x[:, h] for x in xv])
        e_q = G.rel_l2(ref, oa.attend_head(q[:, h], kx, vx, scale=sc, causal=causal))
        G.log(f"attend {name} h{h}: rel-L2 logits {e_log:.3g} (tol {LOGIT_TOL}), out {e_out:.3g} (tol {OUT_TOL}); "
              f"quantized-vs-bf16-cache out {e_q:.3g}")
        assert e_log <= LOGIT_TOL, f"{name} h{h}: logits rel-L2 {e_log}"
        assert e_out <= OUT_TOL, f"{name} h{h}: output rel-L2 {e_out}"


def test_tiny_causal_fp32_queries():
    wl = synth.workload(1)
    _run("tiny", wl, [(0, 1560)], 1560, [0], causal=True, logit_queries=1560)


def test_field_ragged_multi_chunk():
    wl = synth.workload(2, n_heads=2, n_clusters=64)
    _run("field-ragged", wl, [(0, 1000), (1000, 2100), (2100, 2300)], 300, [0, 1])


def test_progressive_three_stages():
    wl = synth.workload(3, n_heads=2, n_clusters=64)
    _run("progressive", wl, [(0, 900), (900, 1700)], 200, [1])


def test_progressive_causal_bf16_queries():
    """Token-causal attention over a three-stage cache with bf16 queries: the
    dense-decode path (every key row decoded once, then the tiles of one fresh
    chunk) under the token-causal mask (frames of one token from key 0)."""
    wl = synth.workload(3, n_heads=2, n_clusters=64)
    _run("progressive-causal", wl, [(0, 700), (700, 1300)], 1300, [0], causal=True, logit_queries=96)


def test_quantwm_psac():
    wl = synth.workload(4, n_heads=2, n_clusters=64)
    _run("quantwm", wl, [(0, 1200), (1200, 2400)], 260, [0, 1])


def test_mixed_precision_keys():
    wl = synth.workload(5, n_heads=2, n_clusters=64)
    _run("mixed", wl, [(0, 1100), (1100, 2000)], 150, [0])


def test_int4_uniform_cache():
    """Uniform INT4 keys and values (one stage, groups of 32), two ragged chunks."""
    wl = synth.workload(2, n_heads=2, n_clusters=64, bits=4)
    _run("int4", wl, [(0, 1000), (1000, 1800)], 200, [0, 1])


def test_int4_two_stage_cache():
    """Uniform INT4 keys and values with two progressive stages (the multi-stage
    INT4 variant of the QVG notes' main table)."""
    wl = synth.workload(3, n_heads=2, n_clusters=32, bits=4, n_stages=2)
    _run("int4-2stage", wl, [(0, 900), (900, 1500)], 130, [1])


def test_single_query():
    wl = synth.workload(2, n_heads=2, n_clusters=16)
    _run("single-query", wl, [(0, 300), (300, 364)], 1, [0, 1], logit_queries=1)


def test_partial_wave_one_tile_cache():
    """33 queries (one full wave of 32 and one query more) over a cache of exactly one 64-key tile."""
    wl = synth.workload(2, n_heads=2, n_clusters=16)
    _run("partial-wave", wl, [(0, 64)], 33, [1], logit_queries=33)


def test_large_logits_rescaling():
    """Queries scaled by 32: logits in the thousands, near one-hot softmax rows, so the
    running maximum keeps growing across tiles (the online rescaling path)."""
    wl = synth.workload(2, n_heads=2, n_clusters=32)
    _run("large-logits", wl, [(0, 700), (700, 1500)], 100, [0, 1], q_scale=32.0)


# Beyond the fp16 range: keys x 2^8 (scales up to ~2.5e4, decoded keys past 6.5e4),
# values x 2^8 (~2.5e5), queries x 2^14 (~8e4); the softmax scale takes the logits
# back to their usual size.  The power-of-two operand scaling must keep every
# result within the usual bars.
BIG = dict(q_scale=2.0 ** 14, kv_scale=(2.0 ** 8, 2.0 ** 8), softmax_scale=2.0 ** -22 / np.sqrt(128.0))


def test_beyond_fp16_range_fast_path():
    wl = synth.workload(2, n_heads=2, n_clusters=32)
    _run("beyond-fp16", wl, [(0, 800), (800, 1300)], 120, [0, 1], **BIG)


def test_beyond_fp16_range_psac():
    """The same with QSAC + PSAC keys: the PSAC coefficients and qU scale with them."""
    wl = synth.workload(4, n_heads=2, n_clusters=32)
    _run("beyond-fp16-psac", wl, [(0, 700), (700, 1400)], 100, [0, 1], **BIG)


def test_beyond_fp16_range_generic_path():
    """Mixed INT4/INT2 keys and two progressive stages (the generic decode)."""
    wl = synth.workload(5, n_heads=2, n_clusters=32, n_stages=2)
    _run("beyond-fp16-generic", wl, [(0, 700), (700, 1300)], 100, [1], **BIG)


def test_bench_shape_sampled_head():
    """The 5 s cache: 32 heads, 6 chunks of 6,240 tokens, 1,560 queries; the
    oracle quantizes two sampled heads of every chunk (packed bytes compared bit
    for bit) and attends over them."""
    wl = synth.workload(2)
    bounds = [wl.chunk_range(c) for c in range(wl.n_chunks)]
    _run("bench-shape", wl, bounds, wl.n_query, [11, 27], logit_queries=64)


def test_progressive_full_cache_sampled_head():
    """Three progressive stages at full shape: 32 heads, 6 chunks of 6,240 tokens,
    C = 256, INT2 g = 32 per stage, 1,560 queries over the whole cache; the oracle
    quantizes two sampled heads of every chunk (three stages each; packed bytes of
    every stage compared bit for bit) and attends."""
    wl = synth.workload(3)
    bounds = [wl.chunk_range(c) for c in range(wl.n_chunks)]
    _run("progressive-full", wl, bounds, wl.n_query, [9, 22], logit_queries=64)


def test_quantwm_full_cache_sampled_head():
    """QSAC-weighted k-means and rank-8 PSAC on the keys at full shape (32 heads,
    6 chunks of 6,240 tokens, C = 256); the oracle quantizes two sampled heads
    (packed bytes and PSAC coefficients compared) and attends."""
    wl = synth.workload(4)
    bounds = [wl.chunk_range(c) for c in range(wl.n_chunks)]
    _run("quantwm-full", wl, bounds, wl.n_query, [13, 29], logit_queries=64)


def test_long_horizon_full_cache_sampled_queries():
    """The one-minute cache at full size: 72 chunks of 6,240 tokens (449,280 keys),
    32 heads, keys mixed INT4 on the 26 most query-sensitive channels / INT2 on the
    rest, values INT2, C = 256; 1,560 queries attend over the whole packed cache.
    The oracle quantizes heads 0 and 23 of every chunk itself (the packed bytes of
    both are compared bit for bit) and attends 65 sampled queries (every 24th) in
    float64; logits of the first 64 queries are checked through the debug path.
    Then one autoregressive step at full size: the last chunk's queries over the 71
    packed chunks before it and its own unquantized keys (frame-block causal),
    65 sampled queries on the same heads."""
    wl = synth.workload(5)
    H, heads, n = wl.n_heads, [0, 23], wl.n_chunks
    t = G.torch()
    kcfg, vcfg = G.config_of(wl, "K"), G.config_of(wl, "V")
    hist = synth.history_queries(wl)
    perm = np.stack([ops.sensitivity_perm(ops.qsac_weights(hist[:, j]), wl.n_int4) for j in range(H)])
    pd = t.from_numpy(perm.astype(np.uint8)).to(G.dev())
    ntok = [b - a for a, b in (wl.chunk_range(c) for c in range(n))]
    ws = G.workspace(kcfg, max(ntok), wl.n_query, n)
    wsv = G.workspace(vcfg, max(ntok))
    kch, vch, xk0, xv0 = [None] * n, [None] * n, [None] * n, [None] * n
    G.log(f"long-horizon: generating and quantizing {n} chunks x 2 tensors")
    last = None
    for c, out in G.generated_chunks(5, n, heads):
        (kb, xk0[c]), (vb, xv0[c]) = out["K"], out["V"]
        kd = t.from_numpy(kb.view(np.int16)).to(G.dev()).view(t.bfloat16)
        vd = t.from_numpy(vb.view(np.int16)).to(G.dev()).view(t.bfloat16)
        kch[c] = G.quantize(kcfg, kd, perm=pd, ws=ws)
        vch[c] = G.quantize(vcfg, vd, ws=wsv)
        if c == n - 1:
            last = (kd, vd)                      # the fresh chunk of the autoregressive step below
        del kd, vd
    q = synth.queries(wl)
    qd = G.to_dev(q, wl.dtype)
    out = t.empty((wl.n_query, H, 128), dtype=t.float32, device=G.dev())
    G.log(f"long-horizon: attend Nq={wl.n_query} over Nk={sum(ntok)}")
    qk.qkv_attend(kcfg, vcfg, qd, kch, vch, ntok, out, ws)
    nl = 64
    logits = t.empty((H, nl, sum(ntok)), dtype=t.float32, device=G.dev())
    out_l = t.empty((nl, H, 128), dtype=t.float32, device=G.dev())
    qk.qkv_attend(kcfg, vcfg, qd[:nl].contiguous(), kch, vch, ntok, out_l, ws, logits=logits)
    o_all = out.cpu().numpy()
    lg_all = {h: logits[h].cpu().numpy() for h in heads}
    del logits
    G.log(f"long-horizon: oracle on heads {heads} ({2 * n * len(heads)} problems)")
    jobs = []
    for c in range(n):
        for hi, h in enumerate(heads):
            jobs.append((xk0[c][:, hi], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group,
                                             iters=wl.kmeans_iters, n_int4=kcfg.n_int4_channels, perm=perm[h])))
            jobs.append((xv0[c][:, hi], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group,
                                             iters=wl.kmeans_iters)))
    res = G.oracle_problems(jobs)

    def job(c, hi, ti):
        return res[(c * len(heads) + hi) * 2 + ti]

    near = 0
    for c in range(n):
        for ti, (tensor, chunks, cfg) in enumerate((("K", kch, kcfg), ("V", vch, vcfg))):
            near += G.compare_chunk(f"long-horizon chunk {c} {tensor}", wl, tensor, xk0[c], chunks[c], cfg,
                                    {h: job(c, hi, ti) for hi, h in enumerate(heads)}, heads)
    G.log(f"long-horizon: packed K/V bit-exact on heads {heads} of all {n} chunks (near-ties {near})")
    sample = np.arange(0, wl.n_query, 24)
    for hi, h in enumerate(heads):
        k_hat = np.concatenate([job(c, hi, 0).x_hat for c in range(n)])
        v_hat = np.concatenate([job(c, hi, 1).x_hat for c in range(n)])
        ref = oa.attend_head(q[sample, h], k_hat, v_hat)
        e_out = G.rel_l2(o_all[sample, h], ref)
        e_log = G.rel_l2(lg_all[h], oa.logits(q[:nl, h], k_hat))
        G.log(f"long-horizon h{h}: rel-L2 logits {e_log:.3g} (tol {LOGIT_TOL}), out {e_out:.3g} (tol {OUT_TOL}) "
              f"on {len(sample)} sampled queries over {k_hat.shape[0]} keys")
        assert e_log <= LOGIT_TOL, f"long-horizon h{h}: logits rel-L2 {e_log}"
        assert e_out <= OUT_TOL, f"long-horizon h{h}: output rel-L2 {e_out}"
    # one autoregressive step at full size: the last chunk's 6,240 queries over the 71
    # packed chunks before it plus its own bf16 keys and values (frame-block causal)
    c = n - 1
    qf = synth.chunk_queries(wl, c)
    qfd = G.to_dev(qf, "bf16")
    ws_f = G.workspace(kcfg, max(ntok), ntok[c], c)
    out_f = t.empty((ntok[c], H, 128), dtype=t.float32, device=G.dev())
    G.log(f"long-horizon AR step: {c} cached chunks + a fresh chunk of {ntok[c]} tokens")
    qk.qkv_attend_fresh(kcfg, vcfg, qfd, kch[:c], vch[:c], ntok[:c], last[0], last[1], wl.tokens_per_frame, out_f, ws_f)
    of = out_f.cpu().numpy()
    sample = np.arange(0, ntok[c], 96)
    for hi, h in enumerate(heads):
        k_hat = np.concatenate([job(cc, hi, 0).x_hat for cc in range(c)])
        v_hat = np.concatenate([job(cc, hi, 1).x_hat for cc in range(c)])
        ref = oa.attend_fresh(qf[sample, h], k_hat, v_hat, xk0[c][:, hi], xv0[c][:, hi], wl.tokens_per_frame,
                              q_index=sample)
        e = G.rel_l2(of[sample, h], ref)
        G.log(f"long-horizon AR step h{h}: output rel-L2 {e:.3g} on {len(sample)} sampled queries (tol {OUT_TOL})")
        assert e <= OUT_TOL, f"long-horizon AR step h{h}: output rel-L2 {e}"


def test_layers_stacked_as_heads():
    """Per-layer batching: every step of the path is independent per head, so L
    layers that share a configuration stack along the head axis -- one quantize
    call per chunk and one attention launch for all of them.  Here 4 layers of 4
    heads (16 stacked heads) over two ragged chunks: each layer's heads in the
    stacked packed chunks equal the layer quantized alone, byte for byte, and
    each layer's outputs, from the stacked launch and from the layer's own
    launch, match the oracle on sampled heads."""
    t = G.torch()
    L, Hl = 4, 4
    wl = synth.workload(2, n_heads=L * Hl, n_clusters=64, frames=2)
    bounds = [(0, 1400), (1400, 3120)]
    nq = 200
    cfg_s, cfg_l = G.config_of(wl, "K"), G.config_of(wl, "K", n_heads=Hl)
    xs = {tensor: [synth.kv_tokens(wl, tensor, a, b) for a, b in bounds] for tensor in ("K", "V")}
    ntok = [b - a for a, b in bounds]
    ws_s = G.workspace(cfg_s, max(ntok), nq, len(bounds))
    ws_l = G.workspace(cfg_l, max(ntok), nq, len(bounds))
    packs_s = {tn: [] for tn in ("K", "V")}
    packs_l = {tn: [[] for _ in range(L)] for tn in ("K", "V")}
    for tensor in ("K", "V"):
        for ci, x in enumerate(xs[tensor]):
            xd = G.to_dev(x, "bf16")
            packs_s[tensor].append(G.quantize(cfg_s, xd, ws=ws_s))
            for l in range(L):
                packs_l[tensor][l].append(G.quantize(cfg_l, xd[:, l * Hl:(l + 1) * Hl], ws=ws_l))
            vs = G.host_views(packs_s[tensor][ci], cfg_s, ntok[ci])
            for l in range(L):
                vl = G.host_views(packs_l[tensor][l][ci], cfg_l, ntok[ci])
                for key in ("labels", "codes", "scales", "centroids"):
                    assert np.array_equal(vs[key][:, l * Hl:(l + 1) * Hl], vl[key]), \
                        f"{tensor} chunk {ci} layer {l}: stacked {key} differ from the layer alone"
    G.log(f"stacked layers: {L} layers x {Hl} heads quantized in one call per chunk = per-layer calls, byte for byte")
    q = synth.queries(wl, n=nq)
    qd = G.to_dev(q, "bf16")
    out_s = t.empty((nq, L * Hl, 128), dtype=t.float32, device=G.dev())
    qk.qkv_attend(cfg_s, cfg_s, qd, packs_s["K"], packs_s["V"], ntok, out_s, ws_s)
    out_l = []
    for l in range(L):
        o = t.empty((nq, Hl, 128), dtype=t.float32, device=G.dev())
        qk.qkv_attend(cfg_l, cfg_l, qd[:, l * Hl:(l + 1) * Hl], packs_l["K"][l], packs_l["V"][l], ntok, o, ws_l)
        out_l.append(o.cpu().numpy())
    os_ = out_s.cpu().numpy()
    checked = [(0, 1), (1, 2), (3, 3)]               # (layer, head within the layer)
    jobs = [(xs[tensor][ci][:, l * Hl + hl], dict(n_clusters=64, bits=2, group=32, iters=10))
            for l, hl in checked for ci in range(len(bounds)) for tensor in ("K", "V")]
    res = G.oracle_problems(jobs)
    for i, (l, hl) in enumerate(checked):
        r = res[i * 2 * len(bounds): (i + 1) * 2 * len(bounds)]
        k_hat = np.concatenate([r[2 * ci].x_hat for ci in range(len(bounds))])
        v_hat = np.concatenate([r[2 * ci + 1].x_hat for ci in range(len(bounds))])
        ref = oa.attend_head(q[:, l * Hl + hl], k_hat, v_hat)
        e_s, e_l = G.rel_l2(os_[:, l * Hl + hl], ref), G.rel_l2(out_l[l][:, hl], ref)
        G.log(f"stacked layers: layer {l} head {hl}: rel-L2 stacked {e_s:.3g}, per-layer {e_l:.3g} (tol {OUT_TOL})")
        assert e_s <= OUT_TOL and e_l <= OUT_TOL
