"""Throughput of the KV-cache compression hot path on one MI355X.

One step = the whole path over one batch of synthetic input: every chunk of the
cache is quantized (K and V: k-means smoothing, per-group INT2 codes, packing;
the 12 independent problems go through one batched call), then one query chunk
attends over the full packed cache.  Default workload: 32
heads, d = 128, bf16, 6 chunks of 6,240 tokens (37,440 tokens), C = 256,
INT2 with groups of 32, 1,560 queries.

Prints one JSON line.  `value` is KV tokens per second through the whole step
(tokens quantized into the cache and attended, inputs resident in HBM);
per-kernel figures, the roofline of the fused attention kernel (plus the k-means assign
step and quant-pack) and the CPU oracle
baseline are extra fields.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens quantized/s + fused INT2 attention TFLOP/s, GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
MAX_BATCH = 16         # problems per qkv_quantize_chunks call
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=2, help="workload id (2: 5 s cache, 3, 4, 5)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--copy-calibration", action="store_true",
                   help="first copy 256 MiB device to device once (reference kernel for HBM byte counters)")
    return p.parse_args()


def stored_traffic(kernel: str, sources) -> dict | None:
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if the
    kernel's sources are unchanged since the counters were taken (else None)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic_c2_bench_step.md")
    try:
        text = open(path).read()
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cid: int) -> dict:
    """Time the oracle (single process, one BLAS/OpenMP thread) on a bounded
    sample: head 0's K and V problems of chunk 0, and one head's attention over a
    cache of the workload's length; extrapolated to the workload's step."""
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    code = f"""
import json, time, numpy as np, sys
sys.path.insert(0, {ROOT!r})
from video_model_kv_amd import synth
from oracle import pipeline, attention
wl = synth.workload({cid})
tq, hats = 0.0, []
for tensor in ('K', 'V'):
    x = synth.kv_chunk(wl, tensor, 0, heads=[0])[:, 0]
    t0 = time.perf_counter()
    res = pipeline.quantize_problem(x, wl.n_clusters, wl.bits, wl.group, wl.n_stages, wl.kmeans_iters)
    tq += time.perf_counter() - t0
    hats.append(res.x_hat)
reps = -(-wl.n_tokens // x.shape[0])
k_hat = np.concatenate([hats[0]] * reps)[:wl.n_tokens]
v_hat = np.concatenate([hats[1]] * reps)[:wl.n_tokens]
q = synth.queries(wl, heads=[0])[:, 0]
t0 = time.perf_counter()
attention.attend_head(q, k_hat, v_hat)
ta = time.perf_counter() - t0
print(json.dumps(dict(tq=tq / 2, ta=ta, n=x.shape[0])))
"""
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    if out.returncode != 0:
        raise RuntimeError("cpu baseline failed: " + out.stderr[-2000:])
    r = json.loads(out.stdout.strip().splitlines()[-1])
    from video_model_kv_amd import synth
    wl = synth.workload(cid)
    problems = 2 * wl.n_heads * wl.n_chunks
    step_s = problems * r["tq"] + wl.n_heads * r["ta"]
    return {"value": wl.n_tokens / step_s, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"head 0's K and V problems of chunk 0 ({r['n']} tokens each, full k-means + quantize: "
                       f"{r['tq']:.2f} s per problem) and one head's float64 attention over {wl.n_tokens} keys "
                       f"({r['ta']:.2f} s), extrapolated to {problems} problems + {wl.n_heads} heads per step")}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import video_model_kv_amd as qk
    from video_model_kv_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qk.lib()
    dev = torch.device("cuda")
    wl = synth.workload(a.workload)
    H, d = wl.n_heads, 128

    def cfg_of(tensor):
        mixed = tensor == "K" and wl.n_int4 > 0
        return qk.Config(n_heads=H, n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group,
                         n_stages=wl.n_stages, kmeans_iters=wl.kmeans_iters,
                         n_int4_channels=wl.n_int4 if mixed else 0,
                         psac_rank=wl.psac_rank if tensor == "K" else 0,
                         use_qsac=1 if (wl.qsac and tensor == "K") else 0)

    kcfg, vcfg = cfg_of("K"), cfg_of("V")
    log(f"workload {wl.name}: H={H} chunks={wl.n_chunks} x {wl.chunk_tokens} tokens, C={wl.n_clusters}, "
        f"stages={wl.n_stages}, Nq={wl.n_query}")
    # ---- inputs, resident in HBM ----
    t0 = time.time()
    xk, xv, ntok = [], [], []
    for c in range(wl.n_chunks):
        for tensor, lst in (("K", xk), ("V", xv)):
            x = synth.kv_chunk(wl, tensor, c)
            lst.append(torch.from_numpy(x).to(torch.bfloat16).to(dev))
        ntok.append(xk[-1].shape[0])
    q = torch.from_numpy(synth.queries(wl)).to(torch.bfloat16).to(dev)
    side_k = {}
    ws_fit = None
    if wl.qsac or wl.psac_rank or wl.n_int4:
        hist = torch.from_numpy(synth.history_queries(wl)).to(torch.bfloat16).to(dev)
        ws_fit = torch.empty(qk.qkv_workspace_bytes(kcfg, 0, hist.shape[0], 0), dtype=torch.uint8, device=dev)
        U = torch.empty((H, d, max(wl.psac_rank, 1)), dtype=torch.float32, device=dev)
        w = torch.empty((H, d), dtype=torch.float32, device=dev)
        perm = torch.empty((H, d), dtype=torch.uint8, device=dev)
        qk.qkv_psac_fit(hist, H, wl.psac_rank, wl.n_int4, ws_fit, U_out=U if wl.psac_rank else None,
                        w_out=w, perm_out=perm if wl.n_int4 else None)
        side_k = dict(w=w if wl.qsac else None, perm=perm if wl.n_int4 else None, U=U if wl.psac_rank else None)
    log(f"inputs ready in {time.time() - t0:.1f} s")
    if a.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    maxn = max(ntok)
    ws_bytes = max(qk.qkv_workspace_bytes(kcfg, maxn, wl.n_query, wl.n_chunks), qk.qkv_workspace_bytes(vcfg, maxn))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kp = [torch.empty(qk.qkv_chunk_layout(kcfg, n).bytes, dtype=torch.uint8, device=dev) for n in ntok]
    vp = [torch.empty(qk.qkv_chunk_layout(vcfg, n).bytes, dtype=torch.uint8, device=dev) for n in ntok]
    out = torch.empty((wl.n_query, H, d), dtype=torch.float32, device=dev)
    # The chunk quantizations of a step are independent: K and V of every chunk
    # go through qkv_quantize_chunks in batches of up to MAX_BATCH problems of
    # equal token count, one workspace slice each.
    ks = (side_k.get("w"), side_k.get("perm"), side_k.get("U")) if side_k else None
    problems = [(kcfg, xk[c], kp[c], ks) for c in range(wl.n_chunks)] + \
               [(vcfg, xv[c], vp[c], None) for c in range(wl.n_chunks)]
    batches = []
    for n in sorted(set(ntok)):
        same = [p for p in problems if p[1].shape[0] == n]
        batches += [same[i:i + MAX_BATCH] for i in range(0, len(same), MAX_BATCH)]
    qws = torch.empty(max(qk.qkv_quantize_chunks_workspace_bytes(kcfg, b[0][1].shape[0], len(b)) for b in batches),
                      dtype=torch.uint8, device=dev)

    def quantize_all():
        for b in batches:
            qk.qkv_quantize_chunks([p[0] for p in b], [p[1] for p in b], [p[2] for p in b], qws,
                                   sides=[p[3] for p in b])

    def quantize_one_chunk():        # streaming use: K and V of one new chunk in one call
        qk.qkv_quantize_chunks([kcfg, vcfg], [xk[0], xv[0]], [kp[0], vp[0]], qws, sides=[ks, None])

    def attend():
        qk.qkv_attend(kcfg, vcfg, q, kp, vp, ntok, out, ws, U=side_k.get("U"))

    def step():
        quantize_all()
        attend()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({a.warmup} steps)")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record()
    for i in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / a.steps
    log(f"timed {a.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / a.steps:.3f} ms/step)")

    # ---- per-component and per-kernel timing (events on the launch stream) ----
    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = a.kernel_reps
    t_quant = timed(quantize_all, max(1, reps // 2))
    t_chunk = timed(quantize_one_chunk, max(1, reps // 2))
    t_att = timed(attend, reps)
    # the dominant kernels of the quantizer: one k-means assign (all heads, one
    # tensor) and one quant-pack, through their step-level entry points
    cent = torch.empty((H, wl.n_clusters, d), dtype=torch.float32, device=dev)
    stride = ntok[0] // wl.n_clusters
    cent.copy_(xk[0][0:wl.n_clusters * stride:stride].float().transpose(0, 1))   # strided init rows
    # the labels live in the packed chunk's own label section, so the
    # quant-pack call copies none (its launches: centroid rounding + pack)
    lay0 = qk.qkv_chunk_layout(kcfg, ntok[0])
    labels = kp[0][lay0.off_labels:lay0.off_labels + H * ntok[0]]
    t_assign = timed(lambda: qk.qkv_kmeans_assign(kcfg, xk[0], cent, labels, ws), reps)
    t_pack = timed(lambda: qk.qkv_quant_pack(kcfg, xk[0], labels, cent, kp[0], 0,
                                             perm=side_k.get("perm")), reps)
    n_assign = 2 * wl.n_chunks * wl.kmeans_iters * wl.n_stages
    nk = sum(ntok)
    att_flops = 4.0 * wl.n_query * nk * d * H + (2.0 * wl.n_query * nk * wl.psac_rank * H)
    assign_flops = 2.0 * ntok[0] * wl.n_clusters * d * H
    elems = ntok[0] * H * d
    groups = qk.qkv_chunk_layout(kcfg, ntok[0]).groups_per_token
    words = qk.qkv_chunk_layout(kcfg, ntok[0]).words_per_token
    pack_bytes = elems * 2 + ntok[0] * H * (1 + 4 * words + 2 * groups)
    comp = {
        "quantize_all_ms": t_quant, "attend_ms": t_att,
        "attend_tflops": att_flops / (t_att * 1e-3) / 1e12,
        "kmeans_assign_ms": t_assign, "kmeans_assign_tflops": assign_flops / (t_assign * 1e-3) / 1e12,
        "kmeans_assign_launches_per_step": n_assign,
        "quant_pack_ms": t_pack, "quant_pack_gbps": pack_bytes / (t_pack * 1e-3) / 1e9,
        "kv_tokens_quantized_per_s": nk / (t_quant * 1e-3),
        "quantize_batches_per_step": len(batches),
        "one_chunk_kv_ms": t_chunk, "one_chunk_kv_tokens_per_s": ntok[0] / (t_chunk * 1e-3),
    }
    # Roofline of the fused attention (the metric's headline kernel, MFMA-bound), timed at call level:
    # the qkv_attend call is k_attend plus three small helpers (chunk upload, tile table, split merge,
    # ~3 % of the call; the rocprofv3 summary in profiles/ lists each).  The k-means assign step is
    # reported beside it (its call is k_prep + k_assign).
    achieved = att_flops / (t_att * 1e-3) / 1e12
    tr = stored_traffic("k_attend", ["video_model_kv_amd/csrc/attend.hip", "video_model_kv_amd/csrc/common.h",
                                     "video_model_kv_amd/csrc/kernels.h", "video_model_kv_amd/csrc/layout.h"])
    roof = {"kernel": "k_attend (qkv_attend call)", "bound": "mfma", "achieved": achieved,
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
            "traffic": None if tr is None else tr["read"] + tr["write"],
            "traffic_read_bytes": None if tr is None else tr["read"],
            "traffic_write_bytes": None if tr is None else tr["write"],
            "algorithmic_per_launch": att_flops}
    achieved_a = assign_flops / (t_assign * 1e-3) / 1e12
    assign_roof = {"kernel": "k_assign (qkv_kmeans_assign call)", "bound": "mfma", "achieved": achieved_a,
                   "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved_a / BF16_PEAK_TFLOPS,
                   "traffic": None, "algorithmic_per_launch": assign_flops}
    trq = stored_traffic("k_quant_pack_tile", ["video_model_kv_amd/csrc/quant.hip", "video_model_kv_amd/csrc/common.h",
                                               "video_model_kv_amd/csrc/kernels.h", "video_model_kv_amd/csrc/layout.h"])
    pack_roof = {"kernel": "k_quant_pack_tile (qkv_quant_pack call: k_centroid_bf16 + k_quant_pack_tile)",
                 "bound": "hbm", "achieved": comp["quant_pack_gbps"], "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": comp["quant_pack_gbps"] / HBM_PEAK_GBS,
                 "traffic": None if trq is None else trq["read"] + trq["write"],
                 "algorithmic_per_launch": pack_bytes}
    cpu = None
    if not a.no_cpu_baseline:
        try:
            log("timing the CPU oracle sample")
            cpu = cpu_baseline(a.workload)
        except Exception as e:  # reported, never fatal to the GPU measurement
            log(f"cpu baseline failed: {e}")
    rec = {
        "metric": METRIC, "value": nk / (ms_step * 1e-3), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "heads": H, "head_dim": d, "chunks": wl.n_chunks,
                   "chunk_tokens": wl.chunk_tokens, "cache_tokens": nk, "clusters": wl.n_clusters,
                   "kmeans_iters": wl.kmeans_iters, "stages": wl.n_stages, "bits": wl.bits, "group": wl.group,
                   "int4_channels": wl.n_int4, "psac_rank": wl.psac_rank, "qsac": wl.qsac,
                   "n_query": wl.n_query, "parallelism": "single-gpu"},
        "roofline": roof, "roofline_kmeans_assign": assign_roof, "roofline_quant_pack": pack_roof,
        "components": comp, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
