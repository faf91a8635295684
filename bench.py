"""Throughput of the KV-cache compression hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  1. the history-window statistics the workload uses (qkv_psac_fit: QSAC channel
     weights, PSAC basis, channel ranking of the mixed INT4/INT2 keys);
  2. every chunk of the cache quantized, K and V (k-means smoothing, residual,
     per-group codes, packing; independent problems go through
     qkv_quantize_chunks in batches of up to 16);
  3. one 1,560-query chunk attending over the whole packed cache (qkv_attend).

Default workload: the one-minute cache -- 288 latent frames of 1,560 tokens in
72 chunks of 6,240 (449,280 tokens), 32 heads, d = 128, bf16; keys INT4 on the
26 most query-sensitive channels and INT2 on the rest, values INT2, C = 256,
groups of 32.  The 5 s, progressive and QuantWM caches are timed after it
(fewer steps) and reported under "workloads".  Beside the step, "ar_rollout"
times one autoregressive rollout over the same 72 chunks: per chunk, its 6,240
queries attend over the packed cache plus its own bf16 keys (frame-block
causal), then the chunk is quantized and appended (chunks/s).

Prints one JSON line.  `value` is KV tokens per second through the whole step
(tokens quantized into the cache and attended, inputs resident in HBM).  Extra
fields: per-kernel durations of the step's launches (HIP events recorded by the
library around each launch, in a pass of their own after the timed steps), the
roofline of the step's dominant kernel and of the other hot kernels, the CPU
oracle's throughput on a bounded sample of the same workload, and untimed quality
diagnostics of each workload's cache ("quality": rebuild error against plain
round-to-nearest, attention against the unquantized cache, PSAC's top-1 shift
rate and energy), and the pack kernel on one problem cold and warm ("hbm_cold").
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens quantized/s + fused INT2 attention TFLOP/s, GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 and fp16 MFMA
MAX_BATCH = 16                 # problems per qkv_quantize_chunks call
PROFILE_STEPS = 3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=5, help="headline workload id (2: 5 s cache, 3, 4, 5: one minute)")
    p.add_argument("--extra", default="2,3,4,6",
                   help="workload ids timed after the headline ('' for none; 6: QuantWM with QSAC's range factor)")
    p.add_argument("--batch", type=int, default=16, help="problems per qkv_quantize_chunks call (1-16)")
    p.add_argument("--no-ar", action="store_true", help="skip the autoregressive rollout of the headline workload")
    p.add_argument("--headline-only", action="store_true",
                   help="only the headline step and its kernel timing (no rollout, side measurements or extra workloads)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=5)
    p.add_argument("--copy-calibration", action="store_true",
                   help="first copy 256 MiB device to device once (reference kernel for HBM byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cores() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ---------------------------------------------------------------- inputs
def _gen_chunk(args):
    """Chunk c of workload cid, K and V, as bf16 bit patterns [N, H, 128] (worker process)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from video_model_kv_amd import synth
    cid, c = args
    with threadpool_limits(limits=1):
        wl = synth.workload(cid)
        out = []
        for tensor in ("K", "V"):
            x = synth.kv_chunk(wl, tensor, c)
            out.append((x.view(np.uint32) >> 16).astype(np.uint16))
    return c, out[0], out[1]


def generated_chunks(cid: int, n_chunks: int):
    """(c, K bits, V bits) for every chunk, from a pool of fresh worker processes."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    workers = max(1, min(16, host_cores(), n_chunks))
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        for i, r in enumerate(ex.map(_gen_chunk, [(cid, c) for c in range(n_chunks)])):
            if (i + 1) % 24 == 0:
                log(f"generated {i + 1} / {n_chunks} chunks")
            yield r


class Run:
    """One workload on the device: inputs, packed chunks, workspaces and the step."""

    def __init__(self, cid: int, batch: int):
        import numpy as np
        import torch
        import video_model_kv_amd as qk
        from video_model_kv_amd import synth
        self.qk, self.torch = qk, torch
        dev = torch.device("cuda")
        wl = self.wl = synth.workload(cid)
        H, d = wl.n_heads, 128
        self.kcfg, self.vcfg = self._cfg("K"), self._cfg("V")
        self.ntok = [b - a for a, b in (wl.chunk_range(c) for c in range(wl.n_chunks))]
        xk, xv = [None] * wl.n_chunks, [None] * wl.n_chunks

        def to_dev(bits):
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

        for c, kb, vb in generated_chunks(cid, wl.n_chunks):
            xk[c], xv[c] = to_dev(kb), to_dev(vb)
        self.xk, self.xv = xk, xv
        self.q = torch.from_numpy(synth.queries(wl)).to(torch.bfloat16).to(dev)
        self.stats = wl.qsac or wl.psac_rank > 0 or wl.n_int4 > 0
        self.side = (None, None, None)
        if self.stats:
            self.hist = torch.from_numpy(synth.history_queries(wl)).to(torch.bfloat16).to(dev)
            self.ws_fit = torch.empty(qk.qkv_workspace_bytes(self.kcfg, 0, self.hist.shape[0], 0),
                                      dtype=torch.uint8, device=dev)
            self.U = torch.empty((H, d, max(wl.psac_rank, 1)), dtype=torch.float32, device=dev)
            self.w = torch.empty((H, d), dtype=torch.float32, device=dev)
            self.perm = torch.empty((H, d), dtype=torch.uint8, device=dev)
            self.side = (self.w if wl.qsac else None, self.perm if wl.n_int4 else None,
                         self.U if wl.psac_rank else None)
        maxn = max(self.ntok)
        self.ws = torch.empty(max(qk.qkv_workspace_bytes(self.kcfg, maxn, wl.n_query, wl.n_chunks),
                                  qk.qkv_workspace_bytes(self.vcfg, maxn)), dtype=torch.uint8, device=dev)
        self.kp = [torch.empty(qk.qkv_chunk_layout(self.kcfg, n).bytes, dtype=torch.uint8, device=dev)
                   for n in self.ntok]
        self.vp = [torch.empty(qk.qkv_chunk_layout(self.vcfg, n).bytes, dtype=torch.uint8, device=dev)
                   for n in self.ntok]
        self.out = torch.empty((wl.n_query, H, d), dtype=torch.float32, device=dev)
        # K and V of consecutive chunks in batches of `batch` problems of equal token count
        probs = []
        for c in range(wl.n_chunks):
            probs.append((self.kcfg, xk[c], self.kp[c], self.side))
            probs.append((self.vcfg, xv[c], self.vp[c], None))
        self.batches = []
        for n in sorted(set(self.ntok)):
            same = [p for p in probs if p[1].shape[0] == n]
            self.batches += [same[i:i + batch] for i in range(0, len(same), batch)]
        self.qws = torch.empty(max(qk.qkv_quantize_chunks_workspace_bytes(self.kcfg, b[0][1].shape[0], len(b))
                                   for b in self.batches), dtype=torch.uint8, device=dev)
        self.nk = sum(self.ntok)

    def _cfg(self, tensor):
        wl = self.wl
        mixed = tensor == "K" and wl.n_int4 > 0
        return self.qk.Config(n_heads=wl.n_heads, n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group,
                              n_stages=wl.n_stages, kmeans_iters=wl.kmeans_iters,
                              n_int4_channels=wl.n_int4 if mixed else 0,
                              psac_rank=wl.psac_rank if tensor == "K" else 0,
                              use_qsac=(2 if wl.qsac_range else 1) if (wl.qsac and tensor == "K") else 0)

    def fit(self):
        if self.stats:
            wl = self.wl
            self.qk.qkv_psac_fit(self.hist, wl.n_heads, wl.psac_rank, wl.n_int4, self.ws_fit,
                                 U_out=self.U if wl.psac_rank else None, w_out=self.w,
                                 perm_out=self.perm if wl.n_int4 else None, energy=False)

    def quantize_all(self):
        for b in self.batches:
            self.qk.qkv_quantize_chunks([p[0] for p in b], [p[1] for p in b], [p[2] for p in b], self.qws,
                                        sides=[p[3] for p in b])

    def attend(self):
        self.qk.qkv_attend(self.kcfg, self.vcfg, self.q, self.kp, self.vp, self.ntok, self.out, self.ws,
                           U=self.side[2])

    def step(self):
        self.fit()
        self.quantize_all()
        self.attend()

    # algorithmic work per step of each hot kernel (flops for MFMA kernels, bytes for HBM kernels).
    # The k-means update has no fixed figure: after the first iteration of a
    # bf16 stage it reads only the rows of the tokens whose label changed
    # (data-dependent); its measured HBM bytes are in the rocprofv3 summaries.
    def work_per_step(self) -> dict:
        wl, H, d = self.wl, self.wl.n_heads, 128
        C, iters, L = wl.n_clusters, wl.kmeans_iters, wl.n_stages
        elems = [n * H * d for n in self.ntok]
        att = 4.0 * wl.n_query * self.nk * d * H + 2.0 * wl.n_query * self.nk * wl.psac_rank * H
        assign = sum(2.0 * n * C * d * H for n in self.ntok) * 2 * iters * L
        pack_tile = pack_generic = 0.0
        for cfg in (self.kcfg, self.vcfg):
            lay = self.qk.qkv_chunk_layout(cfg, self.ntok[0])
            for l in range(L):
                esz = 2 if l == 0 else 4
                for n, e in zip(self.ntok, elems):
                    b = e * esz + n * H + H * C * d * 2 + n * H * (4 * lay.words_per_token + 2 * lay.groups_per_token)
                    if l + 1 < L:
                        b += e * 4                            # the next stage's fp32 input
                    if cfg.n_int4_channels > 0:
                        pack_generic += b
                    else:
                        pack_tile += b
        return {"k_attend": ("mfma", att), "k_assign": ("mfma", assign),
                "k_quant_pack_tile": ("hbm", pack_tile), "k_quant_pack": ("hbm", pack_generic)}


def _gen_queries(args):
    """Queries of chunk c's own tokens as bf16 bit patterns (worker process)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from video_model_kv_amd import synth
    cid, c = args
    with threadpool_limits(limits=1):
        q = synth.chunk_queries(synth.workload(cid), c)
    return c, (q.view(np.uint32) >> 16).astype(np.uint16)


def ar_rollout(run: Run) -> dict:
    """One autoregressive rollout over every chunk of the workload: per chunk, the
    chunk's queries attend over the packed cache plus the chunk's own bf16 keys
    and values (frame-block causal), then K and V of the chunk are quantized (one
    qkv_quantize_chunks call) and appended.  Times the whole rollout, and its
    attention and write parts, with events on the launch stream."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    qk, torch, wl = run.qk, run.torch, run.wl
    dev = torch.device("cuda")
    qs = [None] * wl.n_chunks
    workers = max(1, min(16, host_cores(), wl.n_chunks))
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        for c, bits in ex.map(_gen_queries, [(wl.cid, c) for c in range(wl.n_chunks)]):
            qs[c] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    n_max = max(run.ntok)
    ws = torch.empty(qk.qkv_workspace_bytes(run.kcfg, n_max, n_max, wl.n_chunks), dtype=torch.uint8, device=dev)
    qws = torch.empty(qk.qkv_quantize_chunks_workspace_bytes(run.kcfg, n_max, 2), dtype=torch.uint8, device=dev)
    out = torch.empty((n_max, wl.n_heads, 128), dtype=torch.float32, device=dev)
    run.fit()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(wl.n_chunks)]

    def rollout(n, record):
        for c in range(n):
            nf = run.ntok[c]
            if record:
                ev[c][0].record()
            qk.qkv_attend_fresh(run.kcfg, run.vcfg, qs[c], run.kp[:c], run.vp[:c], run.ntok[:c], run.xk[c], run.xv[c],
                                wl.tokens_per_frame, out[:nf], ws, U=run.side[2])
            if record:
                ev[c][1].record()
            qk.qkv_quantize_chunks([run.kcfg, run.vcfg], [run.xk[c], run.xv[c]], [run.kp[c], run.vp[c]], qws,
                                   sides=[run.side, None])
            if record:
                ev[c][2].record()

    rollout(2, False)                            # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rollout(wl.n_chunks, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = ev[0][0].elapsed_time(ev[-1][2]) * 1e-3
    att = sum(e[0].elapsed_time(e[1]) for e in ev) * 1e-3
    wr = sum(e[1].elapsed_time(e[2]) for e in ev) * 1e-3
    d, H = 128, wl.n_heads
    flops = 0.0
    for c in range(wl.n_chunks):            # visible pairs: all cached keys, fresh keys of frames <= own frame
        nf, nc, F = run.ntok[c], sum(run.ntok[:c]), wl.tokens_per_frame
        fresh_pairs = sum(min(nf, (f + 1) * F) * min(F, nf - f * F) for f in range(-(-nf // F)))
        flops += 4.0 * d * H * (nf * nc + fresh_pairs)
    log(f"AR rollout: {wl.n_chunks} chunks in {total:.3f} s ({wl.n_chunks / total:.2f} chunks/s); "
        f"attention {att:.3f} s ({flops / att / 1e12:.0f} TFLOP/s), write path {wr:.3f} s")
    return {"chunks": wl.n_chunks, "seconds": total, "wall_seconds": wall, "chunks_per_s": wl.n_chunks / total,
            "kv_tokens_per_s": run.nk / total, "attend_s": att, "attend_tflops": flops / att / 1e12,
            "attend_flops": flops, "write_s": wr, "write_ms_per_chunk": wr / wl.n_chunks * 1e3,
            "queries_per_step": "the chunk's own tokens", "mask": "frame-block causal over the fresh chunk"}


def temporal_codec(run: Run) -> dict:
    """The practitioner blog's temporally stable codec over the same cache: K and
    V streams of every chunk (4 frames of P positions x H heads) coded in frame
    order with the state carried, then rebuilt to bf16.  Per chunk launch:
    algorithmic bytes = the chunk's input + the state read and written + the
    packed output (coding); packed input + the group's anchor + the bf16 output
    (rebuilding)."""
    qk, torch, wl = run.qk, run.torch, run.wl
    dev = torch.device("cuda")
    P, H, nf = wl.tokens_per_frame, wl.n_heads, wl.chunk_frames
    cfg = qk.TConfig(n_heads=H, frame_tokens=P, bits=2, anchor_every=32, decay=0.8)
    st_bytes = qk.qkv_temporal_state_bytes(cfg)
    states = [torch.empty(st_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    packs, anchors = [], []
    for c in range(wl.n_chunks):
        nb, _ = qk.qkv_temporal_layout(cfg, c * nf, nf)
        packs.append([torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(2)])
    out = torch.empty((nf * P, H, 128), dtype=torch.bfloat16, device=dev)

    def encode_all():
        for c in range(wl.n_chunks):
            for i, x in enumerate((run.xk[c], run.xv[c])):
                qk.qkv_temporal_encode(cfg, x, c * nf, states[i], packs[c][i])

    encode_all()                                   # warm-up (a whole stream: the state restarts at frame 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    encode_all()
    e1.record()
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1)
    # anchors of each chunk's group for rebuilding: chunk c's group anchor is the
    # first frame of chunk 8 * (c // 8) (anchor every 32 frames = 8 chunks)
    def decode_all():
        for c in range(wl.n_chunks):
            a = 8 * (c // 8)
            for i in range(2):
                anchor = packs[a][i]                # the anchor frame's fp16 values lead that chunk's run
                qk.qkv_temporal_decode(cfg, c * nf, nf, packs[c][i], anchor, out)

    decode_all()
    torch.cuda.synchronize()
    e0.record()
    decode_all()
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1)
    n_launch = 2 * wl.n_chunks
    el = nf * P * H * 128                          # elements per chunk and tensor
    coded = P * H * (32 + 4 * 7)                   # bytes per coded frame: codes + 4 x (lo, scale, outlier value, channel)
    anchor_fr = P * H * 128 * 2
    packed_bytes = sum(p[0].numel() for p in packs)
    enc_bytes = n_launch * (el * 2 + 2 * P * H * 128 * 6) + 2 * sum(
        anchor_fr if (c * nf + f) % 32 == 0 else coded for c in range(wl.n_chunks) for f in range(nf))
    dec_bytes = n_launch * (P * H * 128 * 2 + el * 2) + 2 * sum(
        anchor_fr if (c * nf + f) % 32 == 0 else coded for c in range(wl.n_chunks) for f in range(nf))
    res = {"scheme": "practitioner blog: P99 outliers in fp16, per-block min/max INT2, fp16 anchor every 32 frames, "
                     "0.8 error feedback",
           "launches": n_launch, "encode_us_per_chunk": enc_ms * 1e3 / n_launch,
           "decode_us_per_chunk": dec_ms * 1e3 / n_launch,
           "encode_GBps": enc_bytes / (enc_ms * 1e-3) / 1e9, "decode_GBps": dec_bytes / (dec_ms * 1e-3) / 1e9,
           "encode_frac_of_hbm": enc_bytes / (enc_ms * 1e-3) / 8e12, "decode_frac_of_hbm": dec_bytes / (dec_ms * 1e-3) / 8e12,
           "compression_vs_bf16": (wl.n_chunks * el * 2) / packed_bytes}
    log(f"temporal codec: encode {res['encode_us_per_chunk']:.1f} us/chunk ({res['encode_GBps']:.0f} GB/s), "
        f"decode {res['decode_us_per_chunk']:.1f} us/chunk ({res['decode_GBps']:.0f} GB/s), "
        f"{res['compression_vs_bf16']:.2f}x vs bf16")
    return res


def layer_batching(run: Run, n_layers: int = 8, n_chunks: int = 6) -> dict:
    """Per-layer batching: layers stacked along the head axis run as one launch.
    n_layers x n_chunks of the workload's bf16 chunks serve as the layers' caches
    (layer l = chunks l * n_chunks ...), quantized INT2 (C = 256, groups of 32)
    once per layer (32 heads) and once head-stacked (n_layers x 32 heads); the
    attention of the same queries is timed both ways, for the whole query chunk
    and for a small decode-sized one."""
    qk, torch, wl = run.qk, run.torch, run.wl
    dev = torch.device("cuda")
    H = wl.n_heads
    n_layers = min(n_layers, wl.n_chunks // n_chunks)
    cfg_l = qk.Config(n_heads=H, n_clusters=256, bits=2, group=32)
    cfg_s = qk.Config(n_heads=H * n_layers, n_clusters=256, bits=2, group=32)
    ntok = [run.ntok[c] for c in range(n_chunks)]
    n_max = max(ntok)
    ws_l = torch.empty(qk.qkv_workspace_bytes(cfg_l, n_max, wl.n_query, n_chunks), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(qk.qkv_workspace_bytes(cfg_s, n_max, wl.n_query, n_chunks), dtype=torch.uint8, device=dev)

    def packed(cfg, x, ws):
        p = torch.empty(qk.qkv_chunk_layout(cfg, x.shape[0]).bytes, dtype=torch.uint8, device=dev)
        qk.qkv_quantize_chunk(cfg, x, p, ws)
        return p

    kl = [[packed(cfg_l, run.xk[l * n_chunks + c], ws_l) for c in range(n_chunks)] for l in range(n_layers)]
    vl = [[packed(cfg_l, run.xv[l * n_chunks + c], ws_l) for c in range(n_chunks)] for l in range(n_layers)]
    ks, vs = [], []
    for c in range(n_chunks):
        for src, dst in ((run.xk, ks), (run.xv, vs)):
            x = torch.cat([src[l * n_chunks + c] for l in range(n_layers)], dim=1)
            dst.append(packed(cfg_s, x, ws_s))
            del x
    q_s = torch.cat([run.q] * n_layers, dim=1)
    out_l = torch.empty((wl.n_query, H, 128), dtype=torch.float32, device=dev)
    out_s = torch.empty((wl.n_query, H * n_layers, 128), dtype=torch.float32, device=dev)
    res = {"layers": n_layers, "heads_per_layer": H, "chunks_per_layer": n_chunks, "keys_per_layer": sum(ntok)}
    for nq in (wl.n_query, 64):
        def per_layer():
            for l in range(n_layers):
                qk.qkv_attend(cfg_l, cfg_l, run.q[:nq], kl[l], vl[l], ntok, out_l[:nq], ws_l)

        def stacked():
            qk.qkv_attend(cfg_s, cfg_s, q_s[:nq], ks, vs, ntok, out_s[:nq], ws_s)

        tl, ts = timed_call(run, per_layer, 5), timed_call(run, stacked, 5)
        res[f"nq{nq}"] = {"per_layer_launches_ms": tl, "stacked_launch_ms": ts, "speedup": tl / ts}
        log(f"layer batching ({n_layers} layers x {H} heads, {sum(ntok)} keys each), {nq} queries: "
            f"{n_layers} launches {tl:.3f} ms, one stacked launch {ts:.3f} ms ({tl / ts:.2f}x)")
    return res


def time_steps(run: Run, steps: int, warmup: int):
    torch = run.torch
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run.step()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return e0.elapsed_time(e1) / steps, wall


def timed_call(run: Run, fn, reps: int) -> float:
    torch = run.torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def quality(run: Run, n_q: int = 128) -> dict:
    """Quality diagnostics of a workload's packed cache, reported and not targets
    (untimed; the cache of the run's last step):
      - rel-L2 of the rebuilt K and V (all stages, and after each stage) against the
        bf16 input, and the same for plain per-group round-to-nearest (centroids 0,
        QKV_FLAG_RTN), whose ratio is the error reduction of the smoothing (the QVG
        notes' main table, "RTN" row);
      - attention of the first n_q queries over the packed cache against float32
        attention over the unquantized bf16 cache (rel-L2 of the outputs);
      - with PSAC: the top-1 shift rate, the share of (head, query) whose
        highest-logit key differs from that of the exact logits, with the fitted
        U and with U = 0 (the same cache without the correction term), and the
        energy fraction of the fitted subspace (QuantWM summary, second technique)."""
    qk, torch = run.qk, run.torch
    wl, H, d = run.wl, run.wl.n_heads, 128
    run.step()
    torch.cuda.synchronize()
    res = {"queries": n_q, "stages": wl.n_stages}

    def rebuild_err(cfg, xs, packs):
        num = den = 0.0
        for x, pk in zip(xs, packs):
            xh = torch.empty(x.shape, dtype=torch.float32, device=x.device)
            qk.qkv_dequantize(cfg, x.shape[0], pk, xh)
            xf = x.float()
            num += float(((xh - xf) ** 2).sum())
            den += float((xf ** 2).sum())
        return (num / den) ** 0.5

    res["rel_l2_k"] = rebuild_err(run.kcfg, run.xk, run.kp)
    res["rel_l2_v"] = rebuild_err(run.vcfg, run.xv, run.vp)
    if wl.n_stages > 1:
        # stage l quantizes the residual of stages 1 .. l-1 only, so the error after s
        # stages is the rebuild error of an s-stage quantization of the same input
        by_stage = {"k": [], "v": []}
        for s_ in range(1, wl.n_stages):
            for key, cfg0, xs, side in (("k", run.kcfg, run.xk, run.side), ("v", run.vcfg, run.xv, (None, None, None))):
                cfg = dataclasses.replace(cfg0, n_stages=s_)
                packs = []
                for x in xs:
                    pk = torch.empty(qk.qkv_chunk_layout(cfg, x.shape[0]).bytes, dtype=torch.uint8, device=x.device)
                    qk.qkv_quantize_chunk(cfg, x, pk, run.ws, w=side[0], perm=side[1], U=side[2])
                    packs.append(pk)
                by_stage[key].append(rebuild_err(cfg, xs, packs))
                del packs
        res["rel_l2_k_by_stage"] = by_stage["k"] + [res["rel_l2_k"]]
        res["rel_l2_v_by_stage"] = by_stage["v"] + [res["rel_l2_v"]]
    try:
        rk, rv = (dataclasses.replace(c, flags=c.flags | qk.QKV_FLAG_RTN) for c in (run.kcfg, run.vcfg))
        errs = []
        for cfg, xs, side in ((rk, run.xk, run.side), (rv, run.xv, (None, None, None))):
            packs = []
            for x in xs:
                pk = torch.empty(qk.qkv_chunk_layout(cfg, x.shape[0]).bytes, dtype=torch.uint8, device=x.device)
                qk.qkv_quantize_chunk(cfg, x, pk, run.ws, w=side[0], perm=side[1], U=side[2])
                packs.append(pk)
            errs.append(rebuild_err(cfg, xs, packs))
            del packs
        res["rtn_rel_l2_k"], res["rtn_rel_l2_v"] = errs
        res["error_reduction_vs_rtn_k"] = errs[0] / res["rel_l2_k"]
        res["error_reduction_vs_rtn_v"] = errs[1] / res["rel_l2_v"]
    except Exception as e:  # reported, never fatal to the measurement
        res["rtn_error"] = str(e)
    q = run.q[:n_q].contiguous()
    out = torch.empty((n_q, H, d), dtype=torch.float32, device=q.device)
    U = run.side[2]
    nk = run.nk
    logits = torch.empty((H, n_q, nk), dtype=torch.float32, device=q.device) if U is not None else None
    qk.qkv_attend(run.kcfg, run.vcfg, q, run.kp, run.vp, run.ntok, out, run.ws, U=U, logits=logits)
    torch.cuda.synchronize()
    num = den = 0.0
    shift = shift0 = 0
    top_exact = []
    for h in range(H):
        kh = torch.cat([x[:, h] for x in run.xk]).float()
        vh = torch.cat([x[:, h] for x in run.xv]).float()
        qh = q[:, h].float()
        s_exact = torch.matmul(qh, kh.t().contiguous())
        o = torch.matmul(torch.softmax(s_exact / d ** 0.5, dim=1), vh)
        num += float(((out[:, h] - o) ** 2).sum())
        den += float((o ** 2).sum())
        top_exact.append(s_exact.argmax(dim=1))
        if logits is not None:
            shift += int((logits[h].argmax(dim=1) != top_exact[-1]).sum())
    res["attention_rel_l2_vs_bf16_cache"] = (num / den) ** 0.5
    if U is not None:
        qk.qkv_attend(run.kcfg, run.vcfg, q, run.kp, run.vp, run.ntok, out, run.ws, U=torch.zeros_like(U),
                      logits=logits)
        torch.cuda.synchronize()
        for h in range(H):
            shift0 += int((logits[h].argmax(dim=1) != top_exact[h]).sum())
        res["top1_shift_rate_psac"] = shift / (H * n_q)
        res["top1_shift_rate_no_psac"] = shift0 / (H * n_q)
        energy = qk.qkv_psac_fit(run.hist, H, wl.psac_rank, wl.n_int4, run.ws_fit, U_out=U, w_out=run.w,
                                 perm_out=run.perm if wl.n_int4 else None)
        res["psac_energy_mean"] = sum(energy) / len(energy)
        res["psac_energy_min"] = min(energy)
    return res


def hbm_cold(run: Run, reps: int = 10) -> dict:
    """The uniform pack kernel (k_quant_pack_tile, through qkv_quant_pack) on one V
    problem of chunk 0, cold and warm.  Cold: a 512 MB write before each rep evicts
    the 256 MB MALL; the write also keeps the GPU busy while the call is enqueued,
    so the events bracket the kernel alone.  Warm: reps back to back (the
    problem's ~66 MB stay in the MALL).  The step launches the kernel for 8
    problems at once; one problem is the unit the call takes."""
    import statistics
    qk, torch = run.qk, run.torch
    H, d, C = run.wl.n_heads, 128, run.wl.n_clusters
    cfg, x = run.vcfg, run.xv[0]
    n = x.shape[0]
    cent = x[::max(1, n // C)][:C].float().permute(1, 0, 2).contiguous()   # [H][C][d]
    labels = torch.empty((H, n), dtype=torch.uint8, device=x.device)
    qk.qkv_kmeans_assign(cfg, x, cent, labels, run.ws)
    lay = qk.qkv_chunk_layout(cfg, n)
    packed = torch.empty(lay.bytes, dtype=torch.uint8, device=x.device)
    work = n * H * d * 2 + n * H + H * C * d * 2 + n * H * (4 * lay.words_per_token + 2 * lay.groups_per_token)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=x.device)

    def pack():
        qk.qkv_quant_pack(cfg, x, labels, cent, packed)

    cold = []
    for _ in range(reps + 1):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pack()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold = cold[1:]
    warm = timed_call(run, pack, reps)
    del scratch
    cm = statistics.median(cold)
    return {"kernel": "k_quant_pack_tile", "problems_per_launch": 1, "algorithmic_bytes": work,
            "cold_us_median": cm * 1e3, "cold_us_min": min(cold) * 1e3, "warm_us_mean": warm * 1e3,
            "cold_GBps": work / (cm * 1e-3) / 1e9, "warm_GBps": work / (warm * 1e-3) / 1e9}


def kernel_profile(run: Run, steps: int) -> dict:
    """Per-kernel launches and average duration over `steps` steps, from the HIP
    events the library records around its own launches while timing is on."""
    qk, torch = run.qk, run.torch
    torch.cuda.synchronize()
    qk.qkv_timing_enable(True)
    for _ in range(steps):
        run.step()
    torch.cuda.synchronize()
    rec = qk.qkv_timing_read()
    qk.qkv_timing_enable(False)
    return {k: {"launches_per_step": n / steps, "avg_us": ms * 1e3 / n, "ms_per_step": ms / steps}
            for k, (n, ms) in rec.items() if n > 0}


def stored_traffic(profile_file: str, kernel: str, sources) -> dict | None:
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary,
    if the kernel's sources are unchanged since the counters were taken (else None)."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", profile_file)).read()
    except OSError:
        return None
    m = re.search(rf"^traffic {kernel} sha256=([0-9a-f]+) read_bytes=(\d+) write_bytes=(\d+)", text, re.M)
    if not m:
        return None
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != m.group(1):
        return None
    return {"read": int(m.group(2)), "write": int(m.group(3))}


KERNEL_SOURCES = {
    "k_attend": ["attend.hip"], "k_assign": ["kmeans.hip"],
    "k_quant_pack_tile": ["quant.hip"], "k_quant_pack": ["quant.hip"],
}


def rooflines(run: Run, prof: dict, traffic_file: str) -> dict:
    out = {}
    for k, (bound, work) in run.work_per_step().items():
        if k not in prof or work <= 0:
            continue
        p = prof[k]
        per_launch = work / p["launches_per_step"]
        achieved = per_launch / (p["avg_us"] * 1e-6)
        if bound == "mfma":
            achieved, peak, unit = achieved / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            achieved, peak, unit = achieved / 1e9, HBM_PEAK_GBS, "GB/s"
        srcs = ["video_model_kv_amd/csrc/" + s for s in KERNEL_SOURCES[k]] + \
               ["video_model_kv_amd/csrc/" + s for s in ("common.h", "kernels.h", "layout.h")]
        tr = stored_traffic(traffic_file, k, srcs)
        out[k] = {"kernel": k, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                  "frac": achieved / peak, "traffic": None if tr is None else tr["read"] + tr["write"],
                  "traffic_read_bytes": None if tr is None else tr["read"],
                  "traffic_write_bytes": None if tr is None else tr["write"],
                  "algorithmic_per_launch": per_launch, "avg_launch_us": p["avg_us"],
                  "launches_per_step": p["launches_per_step"], "ms_per_step": p["ms_per_step"]}
    return out


# ---------------------------------------------------------------- CPU oracle baseline
def _oracle_problem(args):
    """One (head, tensor) problem through the oracle's write path (worker process, one BLAS thread)."""
    import time as _t
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, ROOT)
    from oracle import pipeline
    x, kw = args
    with threadpool_limits(limits=1):
        t0 = _t.perf_counter()
        res = pipeline.quantize_problem(x, **kw)
        return _t.perf_counter() - t0, res.x_hat


def cpu_baseline(cid: int) -> dict:
    """The oracle on the host cores: one wave of (head, tensor) problems of chunk 0
    in a process pool (one problem per core), and one head's float64 attention of
    64 sampled queries over a cache of the workload's length (BLAS on every core);
    extrapolated to the workload's step."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention, psac
    from video_model_kv_amd import synth
    wl = synth.workload(cid)
    cores = host_cores()
    per_tensor = max(1, cores // 2)
    heads = list(range(min(wl.n_heads, per_tensor)))
    perm = u = w = None
    if wl.qsac or wl.psac_rank or wl.n_int4:
        hist = synth.history_queries(wl, heads=heads)
        wq = [psac.qsac_weights(hist[:, i]) for i in range(len(heads))]
        w = wq if wl.qsac else None
        perm = [psac.sensitivity_perm(x, wl.n_int4) for x in wq] if wl.n_int4 else None
        u = [psac.principal_subspace(psac.query_gram(hist[:, i]), wl.psac_rank)[0]
             for i in range(len(heads))] if wl.psac_rank else None
    jobs = []
    for tensor in ("K", "V"):
        x = synth.kv_chunk(wl, tensor, 0, heads=heads)
        for i in range(len(heads)):
            kw = dict(n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group, n_stages=wl.n_stages,
                      iters=wl.kmeans_iters)
            if tensor == "K":
                kw.update(w=None if w is None else w[i], n_int4=wl.n_int4, perm=None if perm is None else perm[i],
                          u=None if u is None else u[i])
            jobs.append((x[:, i], kw))
    with ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_problem, [(jobs[0][0][:300], dict(jobs[0][1], iters=1))] * len(jobs)))   # start-up
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_problem, jobs))
        t_wave = time.perf_counter() - t0
    k_hat, v_hat = res[0][1], res[len(heads)][1]
    reps = -(-wl.n_tokens // k_hat.shape[0])
    k_all = np.concatenate([k_hat] * reps)[:wl.n_tokens]
    v_all = np.concatenate([v_hat] * reps)[:wl.n_tokens]
    nq = 64
    q = synth.queries(wl, heads=[0])[:nq, 0]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        attention.attend_head(q, k_all, v_all)
        t_att = time.perf_counter() - t0
    problems = 2 * wl.n_heads * wl.n_chunks
    step_s = -(-problems // len(jobs)) * t_wave + t_att * (wl.n_query / nq) * wl.n_heads
    return {"value": wl.n_tokens / step_s, "unit": "KV tokens/s", "cores": len(jobs), "kind": "oracle",
            "sample": (f"one wave of {len(jobs)} (head, tensor) problems of chunk 0 ({k_hat.shape[0]} tokens each, "
                       f"full k-means + quantize, one per process) took {t_wave:.2f} s on {len(jobs)} cores; one "
                       f"head's float64 attention of {nq} queries over {wl.n_tokens} keys took {t_att:.2f} s on "
                       f"{cores} BLAS threads; extrapolated to {problems} problems and {wl.n_query} queries x "
                       f"{wl.n_heads} heads per step ({step_s:.0f} s)")}


# ---------------------------------------------------------------- main
def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import video_model_kv_amd as qk
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qk.lib()
    if a.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    t0 = time.time()
    run = Run(a.workload, a.batch)
    wl = run.wl
    log(f"workload {wl.name}: H={wl.n_heads} chunks={wl.n_chunks} x {wl.chunk_tokens} tokens, C={wl.n_clusters}, "
        f"stages={wl.n_stages}, int4 channels={wl.n_int4}, Nq={wl.n_query}; inputs ready in {time.time() - t0:.1f} s")
    ms_step, wall = time_steps(run, a.steps, a.warmup)
    log(f"timed {a.steps} steps: {ms_step:.3f} ms/step (wall {wall:.3f} ms/step)")
    t_att = timed_call(run, run.attend, a.kernel_reps)
    t_quant = timed_call(run, run.quantize_all, max(1, a.kernel_reps // 2))
    t_fit = timed_call(run, run.fit, a.kernel_reps) if run.stats else 0.0
    prof = kernel_profile(run, PROFILE_STEPS)
    roofs = rooflines(run, prof, f"hbm_traffic_{wl.name}_bench_step.md")
    dominant = max(roofs.values(), key=lambda r: r["ms_per_step"])
    work = run.work_per_step()
    comp = {
        "stats_fit_ms": t_fit, "quantize_all_ms": t_quant, "attend_ms": t_att,
        "attend_tflops": work["k_attend"][1] / (t_att * 1e-3) / 1e12,
        "kv_tokens_quantized_per_s": run.nk / (t_quant * 1e-3),
        "quantize_batches_per_step": len(run.batches), "problems_per_batch": a.batch,
        "kernels": prof,
    }
    lbatch = None
    tcodec = None
    if not a.headline_only:
        try:
            lbatch = layer_batching(run)
        except Exception as e:  # reported, never fatal to the headline measurement
            log(f"layer batching failed: {e}")
        try:
            tcodec = temporal_codec(run)
        except Exception as e:  # reported, never fatal to the headline measurement
            log(f"temporal codec failed: {e}")
    ar = None
    if not a.no_ar and not a.headline_only:
        try:
            ar = ar_rollout(run)
        except Exception as e:  # reported, never fatal to the headline measurement
            log(f"AR rollout failed: {e}")
    cfgd = {"workload": wl.name, "heads": wl.n_heads, "head_dim": 128, "chunks": wl.n_chunks,
            "chunk_tokens": wl.chunk_tokens, "cache_tokens": run.nk, "clusters": wl.n_clusters,
            "kmeans_iters": wl.kmeans_iters, "stages": wl.n_stages, "bits": wl.bits, "group": wl.group,
            "int4_channels": wl.n_int4, "psac_rank": wl.psac_rank, "qsac": wl.qsac, "qsac_range": wl.qsac_range,
            "n_query": wl.n_query, "parallelism": "single-gpu"}
    qual = cold = None
    if not a.headline_only:
        try:
            qual = quality(run)
        except Exception as e:  # reported, never fatal to the GPU measurement
            log(f"quality diagnostics failed: {e}")
        try:
            cold = hbm_cold(run)
        except Exception as e:  # reported, never fatal to the GPU measurement
            log(f"cold pack timing failed: {e}")
    del run
    torch.cuda.empty_cache()

    extras = {}
    for cid in [] if a.headline_only else [int(x) for x in a.extra.split(",") if x.strip()]:
        if cid == a.workload:
            continue
        r = Run(cid, a.batch)
        ms, _ = time_steps(r, max(3, a.steps // 2), 1)
        ta = timed_call(r, r.attend, a.kernel_reps)
        tq = timed_call(r, r.quantize_all, max(2, a.kernel_reps // 2))
        tf = timed_call(r, r.fit, max(2, a.kernel_reps // 2)) if r.stats else 0.0
        w = r.work_per_step()
        extras[r.wl.name] = {"ms_per_step": ms, "value": r.nk / (ms * 1e-3), "unit": "KV tokens/s",
                             "attend_ms": ta, "attend_tflops": w["k_attend"][1] / (ta * 1e-3) / 1e12,
                             "quantize_ms": tq, "fit_ms": tf,
                             "cache_tokens": r.nk, "stages": r.wl.n_stages, "psac_rank": r.wl.psac_rank,
                             "qsac": r.wl.qsac, "qsac_range": r.wl.qsac_range}
        try:
            extras[r.wl.name]["quality"] = quality(r)
        except Exception as e:  # reported, never fatal to the GPU measurement
            log(f"quality diagnostics of {r.wl.name} failed: {e}")
        log(f"extra workload {r.wl.name}: {ms:.3f} ms/step; quantize {tq:.3f} ms, attend {ta:.3f} ms, "
            f"query statistics {tf:.3f} ms")
        del r
        torch.cuda.empty_cache()

    cpu = None
    if not a.no_cpu_baseline:
        try:
            log("timing the CPU oracle sample")
            cpu = cpu_baseline(a.workload)
        except Exception as e:  # reported, never fatal to the GPU measurement
            log(f"cpu baseline failed: {e}")
    rec = {
        "metric": METRIC, "value": cfgd["cache_tokens"] / (ms_step * 1e-3), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp16",
        "dtype_detail": ("K/V/Q bf16 in HBM; k-means distances on bf16 MFMA (fp32 accumulation) with float64 "
                         "re-decision of close calls and exact centroid sums; INT2/INT4 codes with bf16 scales; "
                         "attention on fp16 MFMA with fp32 accumulation and softmax"),
        "data": "synthetic", "config": cfgd,
        "roofline": {k: v for k, v in dominant.items()},
        "rooflines": roofs, "components": comp, "ar_rollout": ar, "temporal_codec": tcodec, "layer_batching": lbatch, "workloads": extras, "quality": qual, "hbm_cold": cold, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
