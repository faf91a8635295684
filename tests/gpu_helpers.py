"""Helpers of the GPU parity tests: device transfer, library calls on synthetic
workloads, and the oracle run per (head, tensor) problem in a process pool.

Only tests import this module.  Inputs come from video_model_kv_amd.synth; the
expected values come from oracle/ alone.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import video_model_kv_amd as qk
from video_model_kv_amd import packed as pk
from oracle import quant as oq


NEAR_TIE = 1e-5


def log(msg: str):
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def dev():
    t = torch()
    if not t.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    qk.lib()      # fail loudly when the HIP library is missing
    return t.device("cuda")


def to_dev(a: np.ndarray, dtype: str = "f32"):
    """float32 numpy values -> device tensor of the workload dtype (bf16 values are exact)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        x = x.to(t.bfloat16)
    return x.to(dev())


def bits16(x) -> np.ndarray:
    """int16 device/host tensor of bf16 bit patterns -> uint16 numpy."""
    return x.cpu().numpy().view(np.uint16)


def f32_bits_to_bf16(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of bf16-exact float32 values."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "value is not bf16-exact"
    return (u >> 16).astype(np.uint16)


def config_of(wl, tensor: str, n_heads=None, rtn=False) -> qk.Config:
    mixed = tensor == "K" and wl.n_int4 > 0
    return qk.Config(n_heads=n_heads or wl.n_heads, n_clusters=wl.n_clusters, bits=wl.bits, group=wl.group,
                     n_stages=wl.n_stages, kmeans_iters=wl.kmeans_iters,
                     n_int4_channels=wl.n_int4 if mixed else 0,
                     psac_rank=wl.psac_rank if tensor == "K" else 0,
                     use_qsac=(2 if wl.qsac_range else 1) if (wl.qsac and tensor == "K") else 0,
                     flags=qk.QKV_FLAG_RTN if rtn else 0)


def workspace(cfg: qk.Config, n_tokens: int, n_query: int = 0, n_chunks: int = 0):
    t = torch()
    nb = qk.qkv_workspace_bytes(cfg, n_tokens, n_query, n_chunks)
    return t.empty(max(nb, 256), dtype=t.uint8, device=dev())


def quantize(cfg: qk.Config, x_dev, w=None, perm=None, u=None, ws=None):
    t = torch()
    n = x_dev.shape[0]
    lay = qk.qkv_chunk_layout(cfg, n)
    packed = t.zeros(lay.bytes, dtype=t.uint8, device=dev())
    ws = workspace(cfg, n) if ws is None else ws
    qk.qkv_quantize_chunk(cfg, x_dev, packed, ws, w=w, perm=perm, U=u)
    return packed


def host_views(packed, cfg: qk.Config, n_tokens: int) -> dict:
    v = pk.views(packed, cfg, n_tokens)
    out = {}
    for k, val in v.items():
        if k == "layout" or val is None:
            out[k] = val
        else:
            out[k] = val.cpu().numpy()
    return out


# ---------------------------------------------------------------- oracle pool
def _oracle_job(args):
    from threadpoolctl import threadpool_limits
    from oracle import pipeline
    x, kw = args
    with threadpool_limits(limits=1):     # one BLAS thread per worker process
        return pipeline.quantize_problem(x, **kw)


def _spawn_pool(workers: int) -> ProcessPoolExecutor:
    """Worker processes started fresh (no state inherited from a process that
    holds GPU and thread-pool handles)."""
    import multiprocessing as mp
    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))


def pool_workers(n_jobs: int) -> int:
    return min(n_jobs, max(1, min(16, len(os.sched_getaffinity(0)))))


def oracle_problems(jobs, workers: int | None = None):
    """Run oracle.pipeline.quantize_problem for each (x [N, d], kwargs) job;
    long batches print a progress line every 16 problems."""
    if len(jobs) == 1:
        return [_oracle_job(jobs[0])]
    out = []
    with _spawn_pool(workers or pool_workers(len(jobs))) as ex:
        for r in ex.map(_oracle_job, jobs):
            out.append(r)
            if len(jobs) > 16 and len(out) % 16 == 0:
                log(f"oracle: {len(out)} / {len(jobs)} problems")
    return out


def gen_chunk_bits(args):
    """Chunk c of workload cid (all heads) as bf16 bit patterns [N, H, d] uint16
    for K and V, plus float32 rows of the kept heads (bf16-exact)."""
    from threadpoolctl import threadpool_limits
    from video_model_kv_amd import synth
    cid, c, keep = args
    with threadpool_limits(limits=1):
        wl = synth.workload(cid)
        out = {}
        for tensor in ("K", "V"):
            x = synth.kv_chunk(wl, tensor, c)
            out[tensor] = ((x.view(np.uint32) >> 16).astype(np.uint16), x[:, keep].copy())
    return c, out


def generated_chunks(cid: int, n_chunks: int, keep):
    """Yields (c, {tensor: (bf16 bits, kept heads)}) in chunk order, generated in
    a process pool, with a progress line every 8 chunks."""
    with _spawn_pool(pool_workers(n_chunks)) as ex:
        for c, out in ex.map(gen_chunk_bits, [(cid, c, keep) for c in range(n_chunks)]):
            if (c + 1) % 8 == 0:
                log(f"generated {c + 1} / {n_chunks} chunks")
            yield c, out


def compare_chunk(name, wl, tensor, x, packed, cfg, res_by_head, heads):
    """Packed chunk on the device against the oracle's results, bit for bit:
    labels, bf16 centroids, codes and scales of every stage for each listed
    head; PSAC coefficients within one bf16 ulp on fewer than 0.1 % of them
    (the float64 dot products of the two sides differ in summation order).
    Returns the number of near-ties (gap < 1e-5) in the oracle's traces."""
    v = host_views(packed, cfg, x.shape[0])
    near = 0
    for h in heads:
        res = res_by_head[h]
        for l, st in enumerate(res.stages):
            if st.trace is not None:
                near += int(sum((g < NEAR_TIE).sum() for g in st.trace.gaps_iter))
            assert np.array_equal(v["labels"][l, h], st.labels.astype(np.uint8)), f"{name} h{h} stage {l}: labels"
            assert np.array_equal(v["centroids"][l, h].view(np.uint16), f32_bits_to_bf16(st.centroids_bf16)), \
                f"{name} h{h} stage {l}: centroids"
            assert np.array_equal(v["codes"][l, h].view(np.uint32), oq.pack_codes(st.q, res.layout)), \
                f"{name} h{h} stage {l}: codes"
            assert np.array_equal(v["scales"][l, h].view(np.uint16), f32_bits_to_bf16(st.scales)), \
                f"{name} h{h} stage {l}: scales"
        if res.coef is not None:
            got = v["psac"][h].view(np.uint16)
            exp = f32_bits_to_bf16(res.coef)
            diff = np.abs(got.astype(np.int32) - exp.astype(np.int32))
            assert diff.max() <= 1 and (diff > 0).mean() < 1e-3, f"{name} h{h}: psac coefficients"
    return near


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
