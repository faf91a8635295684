"""qkv_quantize_chunk_noalloc, the write path for callers that cannot allocate
device memory: it runs on the library's per-device scratch array and must write
exactly what qkv_quantize_chunk writes with a caller workspace."""
import ctypes as ct

import numpy as np
import pytest

import video_model_kv_amd as qk
from video_model_kv_amd import _binding as B
from video_model_kv_amd import packed as pk
from video_model_kv_amd import synth

FAKE = 0x100000            # an aligned address that validation never dereferences


def test_noalloc_rejects_chunks_beyond_the_scratch_array():
    """Three stages of 32 heads x 6,240 tokens need two fp32 residual buffers
    (2 x 102 MB): rejected on the host with QKV_EWORKSPACE, nothing enqueued."""
    cfg = qk.Config(n_heads=32, n_clusters=256, n_stages=3)
    t = B.qkv_tensor(FAKE, B.QKV_BF16, 0, 6240, 32 * 128, 128)
    side = B.qkv_side(None, None, None)
    st = B.lib().qkv_quantize_chunk_noalloc(ct.byref(cfg.c()), ct.byref(t), ct.byref(side), ct.c_void_p(FAKE), None)
    assert st == B.QKV_EWORKSPACE
    assert "scratch" in B.qkv_last_error()


def _case_big():
    wl = synth.workload(2)
    return qk.Config(n_heads=32, n_clusters=256), synth.kv_chunk(wl, "K", 0), None


def _case_small():
    """QSAC + PSAC keys, fewer heads and tokens, fewer clusters."""
    wl = synth.workload(4, n_heads=2, n_clusters=64)
    cfg = qk.Config(n_heads=2, n_clusters=64, psac_rank=8, use_qsac=1)
    return cfg, synth.kv_tokens(wl, "K", 0, 1300), synth.history_queries(wl)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_call():
    """Three calls in a row: the 5 s cache's key chunk (32 heads x 6,240 tokens,
    C = 256), then a smaller QSAC + PSAC chunk (2 heads x 1,300 tokens, C = 64),
    then the first again: each packed chunk equals qkv_quantize_chunk's bytes."""
    import torch
    assert torch.cuda.is_available()
    dev = torch.device("cuda")
    for name, (cfg, x, hist) in (("big", _case_big()), ("small", _case_small()), ("big again", _case_big())):
        print(f"[no-alloc] {name}: H={cfg.n_heads} N={x.shape[0]} C={cfg.n_clusters}", flush=True)
        xd = torch.from_numpy(x).to(torch.bfloat16).to(dev)
        side = {}
        if hist is not None:
            H = cfg.n_heads
            hd = torch.from_numpy(hist).to(torch.bfloat16).to(dev)
            ws_fit = torch.empty(qk.qkv_workspace_bytes(cfg, 0, hist.shape[0], 0), dtype=torch.uint8, device=dev)
            side["U"] = torch.empty((H, 128, 8), dtype=torch.float32, device=dev)
            side["w"] = torch.empty((H, 128), dtype=torch.float32, device=dev)
            qk.qkv_psac_fit(hd, H, 8, 0, ws_fit, U_out=side["U"], w_out=side["w"])
        n = x.shape[0]
        nbytes = qk.qkv_chunk_layout(cfg, n).bytes
        ref = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=dev)
        ws = torch.empty(qk.qkv_workspace_bytes(cfg, n), dtype=torch.uint8, device=dev)
        qk.qkv_quantize_chunk(cfg, xd, ref, ws, **side)
        got = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev)
        qk.qkv_quantize_chunk_noalloc(cfg, xd, got, **side)
        torch.cuda.synchronize()
        # every section of the packed chunk (the alignment padding between them is never written)
        vr, vg = pk.views(ref, cfg, n), pk.views(got, cfg, n)
        for key in ("codes", "scales", "labels", "centroids", "perm", "psac"):
            if vr[key] is not None:
                assert torch.equal(vg[key], vr[key]), f"{name}: {key} of the no-alloc chunk differ"
        print(f"[no-alloc] {name}: every section identical", flush=True)
