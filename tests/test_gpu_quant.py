"""GPU parity of the KV write path (k-means assign/update, quant-pack, the whole
chunk quantizer, dequantization and the query statistics) against the CPU
oracle on seeded synthetic inputs.

Bar: cluster ids, codes, scales, stored centroids and dequantized values are
bit-exact, with no exclusion: the library's screening bound is rigorous and its
float64 near-ties are decided in the definition's own arithmetic, so every
label equals the oracle's.  Near-ties (float64 gap below 1e-5 relative) are
counted and reported.
"""
import numpy as np
import pytest

import video_model_kv_amd as qk
from video_model_kv_amd import synth
from oracle import kmeans as km
from oracle import psac as ops
from oracle import quant as oq
from oracle.numerics import bf16_rne

import gpu_helpers as G

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-5

# (case id, workload id, overrides, tensor, n_tokens or None for a full chunk)
SMALL = [
    ("tiny-K", 1, {}, "K", None),
    ("tiny-V", 1, {}, "V", None),
    ("field-K-ragged", 2, dict(n_heads=2, n_clusters=64), "K", 1500),
    ("field-V-ragged", 2, dict(n_heads=2, n_clusters=64), "V", 1500),
    ("qsac-K", 4, dict(n_heads=2, n_clusters=64), "K", 1300),
    # three centroid blocks (the bf16 sweep pads to an even count) and an odd
    # number of 32-token sub-blocks (the last item computes a spare one)
    ("field-K-96-clusters-odd", 2, dict(n_heads=2, n_clusters=96), "K", 1100),
]


def _inputs(cid, over, tensor, n):
    wl = synth.workload(cid, **over)
    n = n or wl.chunk_tokens
    x = synth.kv_tokens(wl, tensor, 0, n)
    w = None
    if wl.qsac and tensor == "K":
        hist = synth.history_queries(wl)
        w = np.stack([ops.qsac_weights(hist[:, h]) for h in range(wl.n_heads)])
    return wl, x, w


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_assign_and_update_lockstep(case):
    name, cid, over, tensor, n = case
    wl, x, w = _inputs(cid, over, tensor, n)
    H, N, C = wl.n_heads, x.shape[0], wl.n_clusters
    G.log(f"lockstep {name}: H={H} N={N} C={C} dtype={wl.dtype}")
    traces = [km.kmeans(x[:, h], C, wl.kmeans_iters, None if w is None else w[h], track_objective=False)
              for h in range(H)]
    t = G.torch()
    cfg = G.config_of(wl, tensor)
    xd = G.to_dev(x, wl.dtype)
    ws = G.workspace(cfg, N)
    wd = None if w is None else G.to_dev(w)
    labels = t.empty(H * N, dtype=t.uint8, device=G.dev())
    counts = t.empty(H * C, dtype=t.int32, device=G.dev())
    near_total = 0
    for it in range(wl.kmeans_iters):
        cin = np.stack([tr.centroids_in[it] for tr in traces])
        qk.qkv_kmeans_assign(cfg, xd, G.to_dev(cin), labels, ws, w=wd)
        got = labels.cpu().numpy().reshape(H, N)
        for h, tr in enumerate(traces):
            near = tr.gaps_iter[it] < NEAR_TIE
            mism = got[h] != tr.labels_iter[it]
            assert not np.any(mism), f"{name} iter {it} head {h}: {int(mism.sum())} label mismatches " \
                                     f"({int((mism & near).sum())} of them near-ties)"
            near_total += int(near.sum())
        # update from the oracle's labels of this iteration
        lab = np.stack([tr.labels_iter[it] for tr in traces]).astype(np.uint8)
        cd = G.to_dev(cin)
        qk.qkv_kmeans_update(cfg, xd, t.from_numpy(lab.reshape(-1)).to(G.dev()), cd, ws, counts)
        exp = np.stack([tr.centroids_in[it + 1] if it + 1 < wl.kmeans_iters else tr.centroids for tr in traces])
        got_c = cd.cpu().numpy()
        assert np.array_equal(got_c.view(np.uint32), exp.view(np.uint32)), \
            f"{name} iter {it}: {int((got_c != exp).sum())} centroid values differ"
        exp_counts = np.stack([np.bincount(lab[h], minlength=C) for h in range(H)])
        assert np.array_equal(counts.cpu().numpy().reshape(H, C), exp_counts)
    G.log(f"lockstep {name}: every label equal, near-ties (gap < {NEAR_TIE}) among them {near_total}")


def _near_tie_problem(rng, H, N, C):
    """Tokens and centroids of H heads with ties built in.  Per head, C/2
    anchors a_i; tokens are copies of the anchors (some nudged by one bf16 step).
    Centroid pairs around anchor i, by i mod 4:
      0: a + delta and a - delta (delta on a 2^-9 grid, so both are exact):
         equal float64 distances for the anchor's tokens, the lower index wins;
      1: (anchor 0 only) the zero anchor with e and P(e), e of full fp32
         significands over a wide exponent range and P a channel permutation:
         equal real distances, so the float64 rounding of the channel-ordered
         sum decides;
      2: a - delta and a + delta with channel 0 moved by eta, eta from 2^-20
         to 2^-3 over the anchors: relative gaps from ~1e-11 to ~1e-4;
      3: a plus bf16 noise (an ordinary pair)."""
    y = np.zeros((N, H, 128), np.float32)
    c = np.zeros((H, C, 128), np.float32)
    etas = [2.0 ** -e for e in (20, 17, 14, 12, 10, 8, 6, 3)]
    for h in range(H):
        na = C // 2
        a = bf16_rne(rng.standard_normal((na, 128)) * 3.0).astype(np.float32)
        a = np.clip(a, -7.5, 7.5)
        a[1] = 0.0
        for i in range(na):
            delta = (rng.integers(-8, 9, 128) * 2.0 ** -9).astype(np.float32)
            kind = 1 if i == 1 else (i % 4 if i % 4 != 1 else 3)
            if kind == 0:
                c[h, 2 * i], c[h, 2 * i + 1] = a[i] + delta, a[i] - delta
            elif kind == 1:
                e = (rng.standard_normal(128) * 2.0 ** rng.integers(-14, -5, 128)).astype(np.float32)
                c[h, 2 * i], c[h, 2 * i + 1] = e, e[rng.permutation(128)]
            elif kind == 2:
                lo, hi = a[i] - delta, a[i] + delta
                hi[0] = np.float32(hi[0] + np.float32(etas[(i // 4) % len(etas)]))
                c[h, 2 * i], c[h, 2 * i + 1] = lo, hi
            else:
                c[h, 2 * i] = a[i] + bf16_rne(rng.standard_normal(128) * 0.05).astype(np.float32)
                c[h, 2 * i + 1] = a[i] + bf16_rne(rng.standard_normal(128) * 0.05).astype(np.float32)
        pick = rng.integers(0, na, N)
        y[:, h] = a[pick]
        nudge = rng.random(N) < 0.25
        ch = rng.integers(0, 128, N)
        step = np.where(y[np.arange(N), h, ch] == 0, 2.0 ** -20, np.abs(y[np.arange(N), h, ch]) * 2.0 ** -7)
        y[np.arange(N)[nudge], h, ch[nudge]] += (step * rng.choice([-1.0, 1.0], N))[nudge].astype(np.float32)
        y[:, h] = bf16_rne(y[:, h]).astype(np.float32)
    return y, c


@pytest.mark.parametrize("variant", ["bf16", "bf16-weighted", "f32-weighted"])
def test_assign_engineered_near_ties(variant):
    """Assign against the oracle on tokens and centroids built to tie: exact
    float64 ties (lowest index), ties decided by float64 rounding order, and
    gaps from ~1e-11 to ~1e-4 relative around the screening bound.  Every
    label must equal the oracle's, with no exclusion."""
    rng = np.random.default_rng({"bf16": 31, "bf16-weighted": 32, "f32-weighted": 33}[variant])
    H, N, C = 8, 2048, 64
    y, c = _near_tie_problem(rng, H, N, C)
    f32 = variant.startswith("f32")
    if f32:   # fp32 tokens off the bf16 grid for a quarter of them
        off = rng.random((N, H)) < 0.25
        y = np.where(off[..., None], y * np.float32(1.0 + 2.0 ** -12), y).astype(np.float32)
    w = rng.uniform(0.5, 2.0, (H, 128)).astype(np.float32) if "weighted" in variant else None
    t = G.torch()
    cfg = qk.Config(n_heads=H, n_clusters=C, bits=2, group=32, kmeans_iters=1, use_qsac=1 if w is not None else 0)
    yd = G.to_dev(y, "f32" if f32 else "bf16")
    labels = t.empty(H * N, dtype=t.uint8, device=G.dev())
    qk.qkv_kmeans_assign(cfg, yd, G.to_dev(c), labels, G.workspace(cfg, N), w=None if w is None else G.to_dev(w))
    got = labels.cpu().numpy().reshape(H, N)
    ties = rounding = graded = 0
    for h in range(H):
        lab, dist = km.assign(y[:, h], c[h], None if w is None else w[h])
        part = np.sort(dist, axis=1)[:, :2]
        ties += int((part[:, 0] == part[:, 1]).sum())
        rounding += int(((lab % 2 == 1) & (lab // 2 == 1)).sum())
        gap = km.relative_gap(dist, lab, y[:, h], c[h], None if w is None else w[h])
        graded += int(((gap > 0) & (gap < 1e-4)).sum())
        mism = got[h] != lab
        assert not np.any(mism), f"{variant} head {h}: {int(mism.sum())} labels differ from the oracle"
    G.log(f"near-tie assign {variant}: every label equal; exact float64 ties {ties}, "
          f"won by the higher index of a rounding-decided pair {rounding}, gaps in (0, 1e-4) {graded}")
    assert ties > 0 and graded > 0


@pytest.mark.parametrize("case", SMALL + [("mixed-K", 5, dict(n_heads=2, n_clusters=64, frames=1), "K", 1560)],
                         ids=[c[0] for c in SMALL] + ["mixed-K"])
def test_quant_pack_lockstep(case):
    name, cid, over, tensor, n = case
    wl, x, w = _inputs(cid, over, tensor, n)
    H, N, C = wl.n_heads, x.shape[0], wl.n_clusters
    G.log(f"quant_pack {name}: H={H} N={N}")
    rng = np.random.default_rng(7)
    perm = None
    if tensor == "K" and wl.n_int4:
        perm = np.stack([rng.permutation(128) for _ in range(H)])
    # oracle labels/centroids (a few iterations are enough for this step)
    traces = [km.kmeans(x[:, h], C, 3, None if w is None else w[h], track_objective=False) for h in range(H)]
    cfg = G.config_of(wl, tensor)
    t = G.torch()
    lay = qk.qkv_chunk_layout(cfg, N)
    packed = t.zeros(lay.bytes, dtype=t.uint8, device=G.dev())
    lab = np.stack([tr.labels for tr in traces]).astype(np.uint8)
    cent = np.stack([tr.centroids for tr in traces])
    ynext = t.empty((H, N, 128), dtype=t.float32, device=G.dev())
    permd = None if perm is None else t.from_numpy(perm.astype(np.uint8)).to(G.dev())
    qk.qkv_quant_pack(cfg, G.to_dev(x, wl.dtype), t.from_numpy(lab.reshape(-1)).to(G.dev()), G.to_dev(cent),
                      packed, 0, perm=permd, y_next=ynext)
    v = G.host_views(packed, cfg, N)
    yn = ynext.cpu().numpy()
    for h in range(H):
        layout = oq.channel_layout(128, wl.bits, wl.group, cfg.n_int4_channels, None if perm is None else perm[h])
        cbf = bf16_rne(cent[h])
        rows = cbf[lab[h].astype(np.int64)]
        r = (x[:, h] - rows).astype(np.float32)
        q, s = oq.quantize_groups(r, layout)
        assert np.array_equal(v["codes"][0, h].view(np.uint32), oq.pack_codes(q, layout)), f"{name} head {h}: codes"
        assert np.array_equal(v["scales"][0, h].view(np.uint16), G.f32_bits_to_bf16(s)), f"{name} head {h}: scales"
        assert np.array_equal(v["centroids"][0, h].view(np.uint16), G.f32_bits_to_bf16(cbf))
        assert np.array_equal(v["labels"][0, h], lab[h])
        yhat = oq.dequantize(q, s, rows, layout)
        assert np.array_equal(yn[h].view(np.uint32), (x[:, h] - yhat).astype(np.float32).view(np.uint32))
        if perm is not None:
            assert np.array_equal(v["perm"][h], perm[h].astype(np.uint8))


def _half_integer_residuals(bits, n, H, rng):
    """float32 rows whose residuals (centroids all zero) divided by their group
    scale land exactly on half-integers, within 2^-21 of them, or elsewhere:
    each group of 32 has an element of magnitude qmax * S with S a power of
    two, so the stored scale is exactly S.  About 5 % of the groups are all
    zero (S = 0) and 5 % have S = 2^-110 (far below the usual range)."""
    qmax = (1 << (bits - 1)) - 1
    halves = np.arange(-qmax, qmax) + 0.5                      # ..., -0.5, 0.5, ..., qmax - 0.5
    y = np.zeros((n, H, 128), np.float64)
    for g in range(4):
        S = 2.0 ** rng.integers(-3, 4, size=(n, H, 1))
        pick = rng.uniform(size=(n, H, 1))
        S = np.where(pick < 0.05, 0.0, np.where(pick < 0.10, 2.0 ** -110, S))
        kind = rng.integers(0, 4, size=(n, H, 32))
        base = rng.choice(halves, size=(n, H, 32))
        nudge = rng.choice([-1.0, 1.0], size=(n, H, 32)) * 2.0 ** -21
        free = rng.uniform(-qmax, qmax, size=(n, H, 32))
        v = np.where(kind == 0, base, np.where(kind == 1, base + nudge, np.where(kind == 2, base - nudge, free)))
        v[:, :, 0] = qmax * rng.choice([-1.0, 1.0], size=(n, H))
        y[:, :, g * 32:(g + 1) * 32] = v * S
    return y.astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_quant_pack_half_integer_quotients(bits):
    """Quotients r / S exactly on or within 2^-21 of a half-integer: codes follow
    the correctly rounded quotient with ties to even (the oracle's definition)."""
    H, N, C = 2, 300, 4
    rng = np.random.default_rng(11 + bits)
    x = _half_integer_residuals(bits, N, H, rng)
    lab = rng.integers(0, C, size=(H, N)).astype(np.uint8)
    cent = np.zeros((H, C, 128), np.float32)
    cfg = qk.Config(n_heads=H, n_clusters=C, bits=bits, group=32)
    t = G.torch()
    G.log(f"quant_pack half-integer quotients: bits={bits} H={H} N={N}")
    packed = t.zeros(qk.qkv_chunk_layout(cfg, N).bytes, dtype=t.uint8, device=G.dev())
    ynext = t.empty((H, N, 128), dtype=t.float32, device=G.dev())
    qk.qkv_quant_pack(cfg, G.to_dev(x), t.from_numpy(lab.reshape(-1)).to(G.dev()), G.to_dev(cent),
                      packed, 0, y_next=ynext)
    v = G.host_views(packed, cfg, N)
    yn = ynext.cpu().numpy()
    ties = 0
    for h in range(H):
        layout = oq.channel_layout(128, bits, 32, 0, None)
        r = x[:, h].astype(np.float32)
        q, s = oq.quantize_groups(r, layout)
        with np.errstate(invalid="ignore", divide="ignore"):
            ties += int(np.sum(np.abs(r / np.repeat(s, 32, axis=1)) % 1.0 == 0.5))
        assert np.any(s == 0) and np.any((s > 0) & (s < 2.0 ** -96)), "zero and tiny scales present"
        assert np.array_equal(v["codes"][0, h].view(np.uint32), oq.pack_codes(q, layout)), f"bits {bits} head {h}: codes"
        assert np.array_equal(v["scales"][0, h].view(np.uint16), G.f32_bits_to_bf16(s)), f"bits {bits} head {h}: scales"
        yhat = oq.dequantize(q, s, np.zeros_like(r), layout)
        assert np.array_equal(yn[h].view(np.uint32), (r - yhat).astype(np.float32).view(np.uint32))
    assert ties > 1000, "the input should hold many exact half-integer quotients"


def test_quant_pack_large_token_stride():
    """A token stride of 2^23 + 256 elements (beyond the tile kernel's 24-bit
    in-tile offsets) routes to the per-group kernel; codes, scales and
    residuals still match the oracle bit for bit."""
    t = G.torch()
    H, N, C = 2, 300, 16
    ST = (1 << 23) + 256
    rng = np.random.default_rng(23)
    x = bf16_rne(rng.normal(0.0, 1.0, size=(N, H, 128)) * rng.choice([1.0, 40.0], size=(N, H, 1)))
    lab = rng.integers(0, C, size=(H, N)).astype(np.uint8)
    cent = rng.normal(0.0, 1.0, size=(H, C, 128)).astype(np.float32)
    cfg = qk.Config(n_heads=H, n_clusters=C, bits=2, group=32)
    G.log(f"quant_pack large token stride: stride {ST} elements, N={N}, H={H}")
    buf = t.empty((N - 1) * ST + H * 128, dtype=t.bfloat16, device=G.dev())
    y = t.as_strided(buf, (N, H, 128), (ST, 128, 1))
    y.copy_(t.from_numpy(np.ascontiguousarray(x, np.float32)).to(t.bfloat16).to(G.dev()))
    packed = t.zeros(qk.qkv_chunk_layout(cfg, N).bytes, dtype=t.uint8, device=G.dev())
    ynext = t.empty((H, N, 128), dtype=t.float32, device=G.dev())
    qk.qkv_quant_pack(cfg, y, t.from_numpy(lab.reshape(-1)).to(G.dev()), G.to_dev(cent), packed, 0, y_next=ynext)
    v = G.host_views(packed, cfg, N)
    yn = ynext.cpu().numpy()
    del buf, y
    for h in range(H):
        layout = oq.channel_layout(128, 2, 32, 0, None)
        rows = bf16_rne(cent[h])[lab[h].astype(np.int64)]
        r = (x[:, h] - rows).astype(np.float32)
        q, s = oq.quantize_groups(r, layout)
        assert np.array_equal(v["codes"][0, h].view(np.uint32), oq.pack_codes(q, layout)), f"head {h}: codes"
        assert np.array_equal(v["scales"][0, h].view(np.uint16), G.f32_bits_to_bf16(s)), f"head {h}: scales"
        yhat = oq.dequantize(q, s, rows, layout)
        assert np.array_equal(yn[h].view(np.uint32), (x[:, h] - yhat).astype(np.float32).view(np.uint32))


FREE = [
    ("tiny-K", 1, {}, "K", None, False),
    ("tiny-V-rtn", 1, {}, "V", None, True),
    ("field-V", 2, dict(n_heads=2, n_clusters=64), "V", 1500, False),
    ("progressive-K", 3, dict(n_heads=2, n_clusters=64), "K", 1500, False),
    ("quantwm-K", 4, dict(n_heads=2, n_clusters=64), "K", 1300, False),
    ("mixed-K", 5, dict(n_heads=2, n_clusters=64), "K", 1500, False),
    # the mixed-layout tile kernel's other tile shapes: 3 x 21 (63 rows) and 1 x 64 (head, token) rows
    ("mixed-K-3-heads", 5, dict(n_heads=3, n_clusters=64), "K", 1501, False),
    ("mixed-K-1-head", 5, dict(n_heads=1, n_clusters=64), "K", 1300, False),
    ("quantwm-range-K", 6, dict(n_heads=2, n_clusters=64), "K", 1300, False),
    ("quantwm-range-K-2-stages", 6, dict(n_heads=2, n_clusters=64, n_stages=2), "K", 1300, False),
]


def _side(wl, tensor):
    """Oracle-computed side inputs (QSAC weights, PSAC basis, channel order)."""
    w = u = perm = None
    if tensor == "K" and (wl.qsac or wl.psac_rank or wl.n_int4):
        hist = synth.history_queries(wl)
        ws_ = [ops.qsac_weights(hist[:, h]) for h in range(wl.n_heads)]
        if wl.qsac:
            w = np.stack(ws_)
        if wl.psac_rank:
            u = np.stack([ops.principal_subspace(ops.query_gram(hist[:, h]), wl.psac_rank)[0]
                          for h in range(wl.n_heads)]).astype(np.float32)
        if wl.n_int4:
            perm = np.stack([ops.sensitivity_perm(x, wl.n_int4) for x in ws_])
    return w, u, perm


def test_incremental_updates_in_every_certificate_class():
    """Three heads of bf16 values through ten k-means iterations, one per class
    of the head-wide exactness certificate (max over channels of
    emax - emin + ceil(log2 N), N = 1,500): head 0 (38) keeps float64 sums
    incrementally from the second update on; head 2, with one magnitude of
    2^-35 in channel 20, sits exactly at the fixed-point bound (55) and keeps
    64-bit integer sums from the third; head 1, with 2^-100 in channel 9 (112),
    takes the full update every iteration.  Every section of the packed chunk
    and x_hat bit-exact against the oracle."""
    wl = synth.workload(2, n_heads=3, n_clusters=64)
    n = 1500
    x = synth.kv_tokens(wl, "V", 0, n).copy()
    x[700, 1, 9] = np.float32(2.0 ** -100)
    x[900, 2, 20] = np.float32(2.0 ** -35)
    cfg = G.config_of(wl, "V")
    G.log(f"incremental updates: H=3 N={n} C=64, one head per certificate class")
    packed = G.quantize(cfg, G.to_dev(x, wl.dtype))
    jobs = [(x[:, h], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                           iters=wl.kmeans_iters)) for h in range(wl.n_heads)]
    res = dict(enumerate(G.oracle_problems(jobs)))
    G.compare_chunk("incremental", wl, "V", x, packed, cfg, res, range(wl.n_heads))
    t = G.torch()
    out = t.empty((n, wl.n_heads, 128), dtype=t.float32, device=G.dev())
    qk.qkv_dequantize(cfg, n, packed, out)
    o = out.cpu().numpy()
    for h in range(wl.n_heads):
        assert np.array_equal(o[:, h].view(np.uint32), res[h].x_hat.view(np.uint32)), f"h{h}: x_hat"


@pytest.mark.parametrize("case", FREE, ids=[c[0] for c in FREE])
def test_quantize_chunk_free_running(case):
    name, cid, over, tensor, n, rtn = case
    wl = synth.workload(cid, **over)
    n = n or wl.chunk_tokens
    x = synth.kv_tokens(wl, tensor, 0, n)
    w, u, perm = _side(wl, tensor)
    cfg = G.config_of(wl, tensor, rtn=rtn)
    G.log(f"free-running {name}: H={wl.n_heads} N={n} stages={cfg.n_stages} qsac={cfg.use_qsac} "
          f"psac={cfg.psac_rank} int4={cfg.n_int4_channels}")
    t = G.torch()
    packed = G.quantize(cfg, G.to_dev(x, wl.dtype),
                        w=None if w is None else G.to_dev(w),
                        perm=None if perm is None else t.from_numpy(perm.astype(np.uint8)).to(G.dev()),
                        u=None if u is None else G.to_dev(u))
    jobs = [(x[:, h], dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                           iters=wl.kmeans_iters, w=None if w is None else w[h], n_int4=cfg.n_int4_channels,
                           perm=None if perm is None else perm[h],
                           u=None if u is None else u[h].astype(np.float64), rtn=rtn,
                           qsac_range=wl.qsac_range and tensor == "K"))
            for h in range(wl.n_heads)]
    res = dict(enumerate(G.oracle_problems(jobs)))
    near = G.compare_chunk(name, wl, tensor, x, packed, cfg, res, range(wl.n_heads))
    # dequantization, f32 and bf16 outputs
    out = t.empty((n, wl.n_heads, 128), dtype=t.float32, device=G.dev())
    qk.qkv_dequantize(cfg, n, packed, out)
    outb = t.empty((n, wl.n_heads, 128), dtype=t.bfloat16, device=G.dev())
    qk.qkv_dequantize(cfg, n, packed, outb)
    o = out.cpu().numpy()
    ob = outb.view(t.int16).cpu().numpy().view(np.uint16)
    for h in range(wl.n_heads):
        assert np.array_equal(o[:, h].view(np.uint32), res[h].x_hat.view(np.uint32)), f"{name} h{h}: x_hat"
        assert np.array_equal(ob[:, h], G.f32_bits_to_bf16(bf16_rne(res[h].x_hat)))
    err = G.rel_l2(o, x)
    G.log(f"free-running {name}: bit-exact; near-ties in oracle trace {near}; rel-L2(x_hat, x) = {err:.4g}")


# (case id, tokens, clusters, bits, group, dtype, stages, input kind)
DEGENERATE = [
    ("all-zero", 300, 16, 2, 32, "bf16", 1, "zero"),
    ("one-cluster", 300, 1, 2, 32, "bf16", 1, "normal"),
    ("tokens-equal-clusters", 64, 64, 2, 32, "bf16", 1, "normal"),
    ("identical-rows-f32-int4-2-stages", 200, 8, 4, 16, "f32", 2, "constant"),
]


@pytest.mark.parametrize("case", DEGENERATE, ids=[c[0] for c in DEGENERATE])
def test_quantize_degenerate_chunks(case):
    """Degenerate chunks: all-zero data (every scale 0, every distance tied),
    a single cluster, as many tokens as clusters, and identical rows through two
    stages; the packed chunk and its dequantization match the oracle bit for bit."""
    name, n, C, bits, group, dtype, stages, kind = case
    H = 2
    rng = np.random.default_rng(31)
    if kind == "zero":
        x = np.zeros((n, H, 128), np.float32)
    elif kind == "constant":
        x = np.ascontiguousarray(np.broadcast_to(bf16_rne(rng.normal(size=(1, H, 128))), (n, H, 128)), np.float32)
    else:
        x = bf16_rne(rng.normal(size=(n, H, 128)) * rng.choice([1.0, 30.0], size=(n, H, 1)))
    cfg = qk.Config(n_heads=H, n_clusters=C, bits=bits, group=group, n_stages=stages, kmeans_iters=10)
    G.log(f"degenerate {name}: N={n} C={C} bits={bits} group={group} {dtype} stages={stages}")
    t = G.torch()
    packed = G.quantize(cfg, G.to_dev(x, dtype))
    jobs = [(x[:, h], dict(n_clusters=C, bits=bits, group=group, n_stages=stages, iters=10)) for h in range(H)]
    res = dict(enumerate(G.oracle_problems(jobs)))
    G.compare_chunk(name, None, "K", x, packed, cfg, res, range(H))
    out = t.empty((n, H, 128), dtype=t.float32, device=G.dev())
    qk.qkv_dequantize(cfg, n, packed, out)
    o = out.cpu().numpy()
    for h in range(H):
        assert np.array_equal(o[:, h].view(np.uint32), res[h].x_hat.view(np.uint32)), f"{name} h{h}: x_hat"


def test_full_chunk_bench_shape_sampled_heads():
    """The bench workload's chunk (32 heads x 6,240 tokens, C = 256, INT2, g = 32)
    in the bench's launch configuration; the oracle recomputes sampled heads."""
    wl = synth.workload(2)
    t = G.torch()
    for tensor, heads in (("K", [0, 17, 31]), ("V", [5, 31])):
        x = synth.kv_chunk(wl, tensor, 0)
        cfg = G.config_of(wl, tensor)
        G.log(f"bench-shape chunk {tensor}: N={x.shape[0]} H={wl.n_heads}; oracle heads {heads}")
        packed = G.quantize(cfg, G.to_dev(x, "bf16"))
        t.cuda.synchronize()
        jobs = [(x[:, h], dict(n_clusters=wl.n_clusters, bits=2, group=32, iters=10)) for h in heads]
        res = dict(zip(heads, G.oracle_problems(jobs)))
        near = G.compare_chunk(f"bench-{tensor}", wl, tensor, x, packed, cfg, res, heads)
        G.log(f"bench-shape chunk {tensor}: bit-exact on heads {heads}; near-ties {near}")


def test_full_chunk_qsac_range_sampled_heads():
    """QSAC with the residual-range factor on the QuantWM cache's whole first
    key chunk (32 heads x 6,240 tokens, C = 256, PSAC r = 8): the per-stage
    range weights come from the device; the oracle recomputes heads 3 and 29
    (weights, k-means, codes, PSAC coefficients) bit for bit."""
    wl = synth.workload(6)
    x = synth.kv_chunk(wl, "K", 0)
    w, u, _ = _side(wl, "K")
    cfg = G.config_of(wl, "K")
    assert cfg.use_qsac == 2
    heads = [3, 29]
    G.log(f"qsac-range chunk: N={x.shape[0]} H={wl.n_heads}; oracle heads {heads}")
    packed = G.quantize(cfg, G.to_dev(x, "bf16"), w=G.to_dev(w), u=G.to_dev(u))
    G.torch().cuda.synchronize()
    jobs = [(x[:, h], dict(n_clusters=wl.n_clusters, bits=2, group=32, iters=10, w=w[h],
                           u=u[h].astype(np.float64), qsac_range=True)) for h in heads]
    res = dict(zip(heads, G.oracle_problems(jobs)))
    near = G.compare_chunk("qsac-range", wl, "K", x, packed, cfg, res, heads)
    G.log(f"qsac-range chunk: bit-exact on heads {heads}; near-ties {near}")


def test_psac_fit_matches_oracle():
    wl = synth.workload(4)
    hist = synth.history_queries(wl)
    H = wl.n_heads
    G.log(f"psac_fit: n={hist.shape[0]} H={H}")
    t = G.torch()
    cfg = G.config_of(wl, "K")
    ws = G.workspace(cfg, 0, hist.shape[0], 0)
    U = t.empty((H, 128, 8), dtype=t.float32, device=G.dev())
    w = t.empty((H, 128), dtype=t.float32, device=G.dev())
    perm = t.empty((H, 128), dtype=t.uint8, device=G.dev())
    energy = qk.qkv_psac_fit(G.to_dev(hist, "bf16"), H, 8, 26, ws, U_out=U, w_out=w, perm_out=perm)
    Ug, wg, pg = U.cpu().numpy(), w.cpu().numpy(), perm.cpu().numpy()
    worst = 0.0
    for h in range(H):
        m = ops.query_gram(hist[:, h])
        uo, lam, eo = ops.principal_subspace(m, 8)
        wo = ops.qsac_weights(hist[:, h])
        assert np.array_equal(wg[h].view(np.uint32), wo.view(np.uint32)), f"head {h}: weights"
        assert np.array_equal(pg[h], ops.sensitivity_perm(wo, 26).astype(np.uint8)), f"head {h}: perm"
        assert abs(energy[h] - eo) < 1e-6
        dp = np.linalg.norm(Ug[h].astype(np.float64) @ Ug[h].T.astype(np.float64) - uo @ uo.T)
        worst = max(worst, dp)
        assert dp < 1e-4, f"head {h}: projector differs by {dp}"
    G.log(f"psac_fit: weights/perm exact, worst projector difference {worst:.3g}, energy[0] {energy[0]:.4f}")
    # rank 0 without the energy fractions (the mixed layout's channel order, as the one-minute cache
    # takes it): only the diagonal of M is formed, and weights and order are the same bits
    w0 = t.empty((H, 128), dtype=t.float32, device=G.dev())
    p0 = t.empty((H, 128), dtype=t.uint8, device=G.dev())
    assert qk.qkv_psac_fit(G.to_dev(hist, "bf16"), H, 0, 26, ws, w_out=w0, perm_out=p0, energy=False) is None
    assert np.array_equal(w0.cpu().numpy().view(np.uint32), wg.view(np.uint32)), "rank 0: weights"
    assert np.array_equal(p0.cpu().numpy(), pg), "rank 0: channel order"


def test_psac_fit_degenerate_histories():
    """The GPU eigensolver at its edges.  An all-zero history: M = 0, no sweep
    runs, every weight is 0 and the energy fraction is 0 (the total is not
    positive); U is still orthonormal.  A history whose channels are mutually
    orthogonal (each query has one nonzero channel): M is diagonal, already
    converged, so U's columns are the unit vectors of the eight largest
    entries in descending order and the energy is their share of the trace."""
    t = G.torch()
    H, n, r = 2, 512, 8
    cfg = G.config_of(synth.workload(4, n_heads=H), "K")
    ws = G.workspace(cfg, 0, n, 0)
    U = t.empty((H, 128, r), dtype=t.float32, device=G.dev())
    w = t.empty((H, 128), dtype=t.float32, device=G.dev())
    zero = np.zeros((n, H, 128), np.float32)
    energy = qk.qkv_psac_fit(G.to_dev(zero, "bf16"), H, r, 0, ws, U_out=U, w_out=w)
    Ug = U.cpu().numpy().astype(np.float64)
    assert np.all(w.cpu().numpy() == 0.0) and all(e == 0.0 for e in energy)
    for h in range(H):
        assert np.allclose(Ug[h].T @ Ug[h], np.eye(r), atol=1e-6), f"zero history, head {h}: U not orthonormal"
    # one nonzero channel per query: query i of head h has value a[h, i % 128] in channel i % 128
    rng = np.random.default_rng(3)
    amp = rng.choice(np.arange(1, 129), size=(H, 128), replace=True).astype(np.float32) / 16.0
    x = np.zeros((n, H, 128), np.float32)
    for i in range(n):
        x[i, :, i % 128] = amp[:, i % 128]
    energy = qk.qkv_psac_fit(G.to_dev(x, "bf16"), H, r, 0, ws, U_out=U, w_out=w)
    Ug = U.cpu().numpy().astype(np.float64)
    for h in range(H):
        d = (x[:, h].astype(np.float64) ** 2).sum(axis=0)       # diag(M); the bf16 inputs are exact here
        order = sorted(range(128), key=lambda k: (-d[k], k))[:r]
        for b, k in enumerate(order):
            col = Ug[h][:, b]
            assert abs(abs(col[k]) - 1.0) < 1e-6 and np.abs(np.delete(col, k)).max() < 1e-6, (
                f"diagonal history, head {h}: column {b} is not e_{k}")
        assert abs(energy[h] - d[order].sum() / d.sum()) < 1e-6
    G.log("psac_fit: zero and diagonal histories as defined")


def test_psac_fit_clustered_spectrum():
    """The GPU eigensolver where single eigenvectors are ill-defined: per head, the
    history's covariance has eight equal leading eigenvalues (100) in a random
    orthogonal basis and the rest in [1, 10], so the sample Gram M has a leading
    cluster of eight (within about 15 % of each other, some pairs within 0.2 %)
    and a gap of about 7.5x after it.  The rank-8 subspace is then well defined: its projector must match LAPACK's on the same M (float64 of the bf16
    queries), and the energy fraction must match."""
    t = G.torch()
    H, n, r = 4, 2048, 8
    rng = np.random.default_rng(11)
    x = np.empty((n, H, 128), np.float32)
    for h in range(H):
        q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
        lam = np.concatenate([np.full(r, 100.0), rng.uniform(1.0, 10.0, 128 - r)])
        x[:, h] = (rng.standard_normal((n, 128)) * np.sqrt(lam)) @ q.T
    x = synth.round_to(x.astype(np.float64), "bf16")
    cfg = G.config_of(synth.workload(4, n_heads=H), "K")
    ws = G.workspace(cfg, 0, n, 0)
    U = t.empty((H, 128, r), dtype=t.float32, device=G.dev())
    w = t.empty((H, 128), dtype=t.float32, device=G.dev())
    energy = qk.qkv_psac_fit(G.to_dev(x, "bf16"), H, r, 0, ws, U_out=U, w_out=w)
    Ug = U.cpu().numpy().astype(np.float64)
    worst = 0.0
    for h in range(H):
        m = ops.query_gram(x[:, h])
        uo, lam_o, eo = ops.principal_subspace(m, r)
        ev = np.linalg.eigvalsh(m)[::-1]
        assert ev[r - 1] > 5.0 * ev[r], f"head {h}: no gap after the leading cluster"
        assert np.allclose(Ug[h].T @ Ug[h], np.eye(r), atol=1e-5), f"head {h}: U not orthonormal"
        dp = np.linalg.norm(Ug[h] @ Ug[h].T - uo @ uo.T)
        worst = max(worst, dp)
        assert dp < 1e-4, f"head {h}: projector differs by {dp}"
        assert abs(energy[h] - eo) < 1e-6, f"head {h}: energy {energy[h]} against {eo}"
    G.log(f"psac_fit: clustered spectrum, worst projector difference {worst:.3g}")


def _batch_vs_single(problems):
    """problems: list of (cfg, x_dev, (w, perm, u) device tensors or None).
    The batched write path must reproduce every single-problem call byte for byte."""
    t = G.torch()
    n = problems[0][1].shape[0]
    packs = [t.zeros(qk.qkv_chunk_layout(cfg, n).bytes, dtype=t.uint8, device=G.dev()) for cfg, _, _ in problems]
    wsb = qk.qkv_quantize_chunks_workspace_bytes(problems[0][0], n, len(problems))
    ws = t.empty(wsb, dtype=t.uint8, device=G.dev())
    qk.qkv_quantize_chunks([p[0] for p in problems], [p[1] for p in problems], packs, ws,
                           sides=[p[2] for p in problems])
    for i, (cfg, x, side) in enumerate(problems):
        w, perm, u = side if side is not None else (None, None, None)
        single = G.quantize(cfg, x, w=w, perm=perm, u=u)
        t.cuda.synchronize()
        assert t.equal(packs[i], single), f"problem {i}: batched bytes differ from the single call"
        del single
    return packs


def test_quantize_batch_mixed_configs_matches_single():
    """K with QSAC + PSAC, V plain, and K with the mixed INT4 layout in one batch
    (configs differ in everything a batch allows), ragged N."""
    t = G.torch()
    n = 1300
    probs = []
    for cid, tensor in ((4, "K"), (4, "V"), (5, "K")):
        wl = synth.workload(cid, n_heads=2, n_clusters=64)
        x = synth.kv_tokens(wl, tensor, 0, n)
        w, u, perm = _side(wl, tensor)
        side = (None if w is None else G.to_dev(w),
                None if perm is None else t.from_numpy(perm.astype(np.uint8)).to(G.dev()),
                None if u is None else G.to_dev(u))
        probs.append((G.config_of(wl, tensor), G.to_dev(x, wl.dtype), side))
    G.log("batch of 3 mixed configs, N=1300, H=2, C=64")
    _batch_vs_single(probs)


def test_quantize_batch_bench_shape_matches_single():
    """The bench's batch: K and V of all six chunks of the 5 s cache (12 problems,
    32 heads x 6,240 tokens, C = 256) in one call, against single calls (whose
    parity with the oracle the sampled-head test above establishes)."""
    wl = synth.workload(2)
    probs = []
    for c in range(wl.n_chunks):
        for tensor in ("K", "V"):
            probs.append((G.config_of(wl, tensor), G.to_dev(synth.kv_chunk(wl, tensor, c), "bf16"), None))
    G.log(f"bench batch: {len(probs)} problems of N={wl.chunk_tokens}, H={wl.n_heads}")
    _batch_vs_single(probs)


def test_quantize_batch_headline_launch_matches_single():
    """The headline bench's launch: K and V of eight chunks of the one-minute
    cache (16 problems of 32 heads x 6,240 tokens, C = 256; keys in the mixed
    INT4/INT2 layout) in one call -- one assign workgroup per head -- against
    single calls, and one K and one V head of the first chunk against the
    oracle."""
    t = G.torch()
    wl = synth.workload(5)
    _, _, perm = _side(wl, "K")
    pd = t.from_numpy(perm.astype(np.uint8)).to(G.dev())
    probs, x0 = [], {}
    for c in range(8):
        for tensor in ("K", "V"):
            x = synth.kv_chunk(wl, tensor, c)
            if c == 0:
                x0[tensor] = x
            probs.append((G.config_of(wl, tensor), G.to_dev(x, "bf16"), (None, pd, None) if tensor == "K" else None))
    G.log(f"headline batch: {len(probs)} problems of N={wl.chunk_tokens}, H={wl.n_heads}")
    packs = _batch_vs_single(probs)
    for i, (tensor, h) in enumerate((("K", 7), ("V", 26))):
        kw = dict(n_clusters=wl.n_clusters, bits=2, group=32, iters=10)
        if tensor == "K":
            kw.update(n_int4=wl.n_int4, perm=perm[h])
        res = G.oracle_problems([(x0[tensor][:, h], kw)])
        near = G.compare_chunk(f"headline-{tensor}", wl, tensor, x0[tensor], packs[i], probs[i][0], {h: res[0]}, [h])
        G.log(f"headline batch: chunk 0 {tensor} head {h} bit-exact against the oracle; near-ties {near}")


def test_quantize_batch_certificate_classes():
    """Four problems in one call with heads of every exactness class spread over
    them (a head with 2^-100 in one channel is outside both classes; head 2
    with 2^-35 in channel 20 sits at the fixed-point bound), so that the later
    iterations' full updates run from per-problem head lists across several
    problems: bytes equal to single calls, and every head of every problem
    bit-exact against the oracle."""
    wl = synth.workload(2, n_heads=3, n_clusters=64)
    n = 1500
    base = synth.kv_tokens(wl, "V", 0, n)
    plants = ([], [(700, 1, 9, -100)], [(700, 1, 9, -100), (900, 2, 20, -35)],
              [(900, 2, 20, -35), (100, 0, 3, -100)])
    xs = []
    for pl in plants:
        x = base.copy()
        for i, h, k, e in pl:
            x[i, h, k] = np.float32(2.0 ** e)
        xs.append(x)
    cfg = G.config_of(wl, "V")
    G.log("batch of 4 problems, N=1500, H=3, C=64, heads of every certificate class")
    packs = _batch_vs_single([(cfg, G.to_dev(x, wl.dtype), None) for x in xs])
    kw = dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages, iters=wl.kmeans_iters)
    res = G.oracle_problems([(x[:, h], kw) for x in xs for h in range(wl.n_heads)])
    for p, x in enumerate(xs):
        G.compare_chunk(f"classes-{p}", wl, "V", x, packs[p], cfg,
                        {h: res[p * wl.n_heads + h] for h in range(wl.n_heads)}, range(wl.n_heads))


def test_quantize_batch_all_ties_overflow_list():
    """Every token of a problem identical: all centroids tie, every token is a
    close call (more than the workgroup's LDS list holds, so the per-wave
    re-decision runs too).  Ties go to the lowest index, so every label is 0,
    the centroid is the token and the residual is zero: the dequantized chunk
    equals the input exactly."""
    t = G.torch()
    n_prob, H, N = 16, 16, 4096
    cfg = qk.Config(n_heads=H, n_clusters=64, bits=2, group=32, kmeans_iters=2)
    rng = np.random.default_rng(7)
    xs = []
    for p in range(n_prob):
        row = bf16_rne(rng.standard_normal((1, H, 128)) * 3.0).astype(np.float32)
        xs.append(G.to_dev(np.repeat(row, N, axis=0), "bf16"))
    packs = [t.zeros(qk.qkv_chunk_layout(cfg, N).bytes, dtype=t.uint8, device=G.dev()) for _ in range(n_prob)]
    ws = t.empty(qk.qkv_quantize_chunks_workspace_bytes(cfg, N, n_prob), dtype=t.uint8, device=G.dev())
    G.log(f"all-ties batch: {n_prob} problems, H={H}, N={N}, C=64")
    qk.qkv_quantize_chunks([cfg] * n_prob, xs, packs, ws)
    for p in range(n_prob):
        v = G.host_views(packs[p], cfg, N)
        assert not np.any(v["labels"]), f"problem {p}: a tie did not go to index 0"
        out = t.empty((N, H, 128), dtype=t.bfloat16, device=G.dev())
        qk.qkv_dequantize(cfg, N, packs[p], out)
        assert t.equal(out, xs[p]), f"problem {p}: dequantized chunk differs from the input"


def test_quantize_batch_progressive_fp32_stages():
    """Six problems of the progressive cache (K and V of chunks 0-2: 32 heads x
    6,240 tokens, C = 256, three stages) in one call: stages 2 and 3 run on the
    fp32 residuals with the wide update (32 clusters per workgroup, chosen for
    launches of at least six 32-head problems).  Every batched chunk must equal
    the single call (narrow update) byte for byte, and two sampled heads match
    the oracle bit for bit in every stage."""
    wl = synth.workload(3)
    probs, xs = [], []
    for c in range(3):
        for tensor in ("K", "V"):
            x = synth.kv_chunk(wl, tensor, c)
            xs.append((tensor, x))
            probs.append((G.config_of(wl, tensor), G.to_dev(x, "bf16"), None))
    G.log(f"progressive batch: {len(probs)} problems of N={wl.chunk_tokens}, H={wl.n_heads}, 3 stages")
    packs = _batch_vs_single(probs)
    checks = [(0, 20), (5, 3)]          # (problem, head)
    jobs = [(xs[p][1][:, h], dict(n_clusters=wl.n_clusters, bits=2, group=32, n_stages=3, iters=10))
            for p, h in checks]
    res = G.oracle_problems(jobs)
    for (p, h), r in zip(checks, res):
        tensor, x = xs[p]
        near = G.compare_chunk(f"progressive-batch p{p}", wl, tensor, x, packs[p], probs[p][0], {h: r}, [h])
        G.log(f"progressive batch: problem {p} ({tensor}) head {h} bit-exact in all 3 stages; near-ties {near}")
