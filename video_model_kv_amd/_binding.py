"""ctypes binding of libqkv (include/qkv.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors (device memory) where the C function takes device pointers, and raises
``QkvError`` with the library's message on a non-zero status.  No step of the
method runs in Python.  Importing works without a GPU; loading the library
needs libqkv.so, built by ``video_model_kv_amd.build`` (missing -> error).
"""
from __future__ import annotations

import ctypes as ct
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
# QKV_LIB_PATH selects another build of the library (the sanitizer tests load a
# host-only instrumented build this way)
LIB_PATH = os.environ.get("QKV_LIB_PATH") or os.path.join(HERE, "libqkv.so")

QKV_OK, QKV_EINVAL, QKV_EUNSUPPORTED, QKV_EDEVICE, QKV_EWORKSPACE = 0, 1, 2, 3, 4
QKV_F32, QKV_BF16 = 0, 1
QKV_FLAG_RTN = 1

EXPORTED = [
    "qkv_version", "qkv_last_error", "qkv_chunk_layout", "qkv_workspace_bytes",
    "qkv_quantize_chunk", "qkv_dequantize", "qkv_attend", "qkv_psac_fit",
    "qkv_kmeans_assign", "qkv_kmeans_update", "qkv_quant_pack",
    "qkv_quantize_chunks", "qkv_quantize_chunks_workspace_bytes", "qkv_quantize_chunk_noalloc",
    "qkv_timing_enable", "qkv_timing_read", "qkv_attend_fresh",
    "qkv_temporal_layout", "qkv_temporal_state_bytes", "qkv_temporal_encode", "qkv_temporal_decode",
]


class QkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libqkv status {status}: {message}")
        self.status = status


class qkv_config(ct.Structure):
    _fields_ = [(n, ct.c_int32) for n in (
        "head_dim", "n_heads", "n_clusters", "kmeans_iters", "n_stages", "bits", "group",
        "n_int4_channels", "psac_rank", "use_qsac", "flags")]


class qkv_tensor(ct.Structure):
    _fields_ = [("ptr", ct.c_void_p), ("dtype", ct.c_int32), ("reserved", ct.c_int32),
                ("n_tokens", ct.c_int64), ("stride_token", ct.c_int64), ("stride_head", ct.c_int64)]


class qkv_side(ct.Structure):
    _fields_ = [("w", ct.c_void_p), ("perm", ct.c_void_p), ("U", ct.c_void_p)]


class qkv_tcfg(ct.Structure):
    _fields_ = [("n_heads", ct.c_int32), ("frame_tokens", ct.c_int32), ("bits", ct.c_int32),
                ("anchor_every", ct.c_int32), ("decay", ct.c_float)]


class qkv_kernel_time(ct.Structure):
    _fields_ = [("name", ct.c_char * 32), ("launches", ct.c_int64), ("total_ms", ct.c_double)]


class qkv_layout(ct.Structure):
    _fields_ = [("bytes", ct.c_uint64),
                ("off_codes", ct.c_uint64), ("stage_bytes_codes", ct.c_uint64),
                ("off_scales", ct.c_uint64), ("stage_bytes_scales", ct.c_uint64),
                ("off_labels", ct.c_uint64), ("stage_bytes_labels", ct.c_uint64),
                ("off_centroids", ct.c_uint64), ("stage_bytes_centroids", ct.c_uint64),
                ("off_perm", ct.c_uint64), ("off_psac", ct.c_uint64),
                ("words_per_token", ct.c_int32), ("groups_per_token", ct.c_int32),
                ("int4_words", ct.c_int32), ("reserved", ct.c_int32), ("n_tokens", ct.c_int64)]


@dataclass
class Config:
    """Python mirror of qkv_config (see include/qkv.h for each field)."""
    n_heads: int
    n_clusters: int
    bits: int = 2
    group: int = 32
    n_stages: int = 1
    kmeans_iters: int = 10
    n_int4_channels: int = 0
    psac_rank: int = 0
    use_qsac: int = 0
    flags: int = 0
    head_dim: int = 128

    def c(self) -> qkv_config:
        return qkv_config(self.head_dim, self.n_heads, self.n_clusters, self.kmeans_iters,
                          self.n_stages, self.bits, self.group, self.n_int4_channels,
                          self.psac_rank, self.use_qsac, self.flags)


@dataclass
class TConfig:
    """Python mirror of qkv_tcfg (the temporally stable codec; include/qkv.h)."""
    n_heads: int
    frame_tokens: int
    bits: int = 2
    anchor_every: int = 32
    decay: float = 0.8

    def c(self) -> qkv_tcfg:
        return qkv_tcfg(self.n_heads, self.frame_tokens, self.bits, self.anchor_every, self.decay)


_lib = None


def lib():
    """The loaded libqkv (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqkv.so is not built ({LIB_PATH}); run python -m video_model_kv_amd.build")
        # torch ships its own HIP runtime; loading it first makes libqkv bind to
        # that same runtime (one device context per process), where loading
        # libqkv first would map a second HIP/HSA runtime from the ROCm install
        # that then sees no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ct.CDLL(LIB_PATH)
        vp, i32, i64, sz = ct.c_void_p, ct.c_int32, ct.c_int64, ct.c_size_t
        P = ct.POINTER
        L.qkv_version.restype = ct.c_int
        L.qkv_last_error.restype = ct.c_char_p
        L.qkv_chunk_layout.argtypes = [P(qkv_config), i64, P(qkv_layout)]
        L.qkv_workspace_bytes.argtypes = [P(qkv_config), i64, i64, i32, P(sz)]
        L.qkv_quantize_chunk.argtypes = [P(qkv_config), P(qkv_tensor), P(qkv_side), vp, vp, sz, vp]
        L.qkv_dequantize.argtypes = [P(qkv_config), i64, vp, P(qkv_tensor), vp]
        L.qkv_attend.argtypes = [P(qkv_config), P(qkv_config), P(qkv_tensor), P(vp), P(vp), P(i64), i32,
                                 vp, i32, ct.c_float, P(qkv_tensor), vp, vp, sz, vp]
        L.qkv_psac_fit.argtypes = [P(qkv_tensor), i32, i32, i32, vp, vp, vp, P(ct.c_float), vp, sz, vp]
        L.qkv_kmeans_assign.argtypes = [P(qkv_config), P(qkv_tensor), vp, vp, vp, vp, sz, vp]
        L.qkv_kmeans_update.argtypes = [P(qkv_config), P(qkv_tensor), vp, vp, vp, vp, sz, vp]
        L.qkv_quant_pack.argtypes = [P(qkv_config), P(qkv_tensor), vp, vp, vp, vp, i32, vp, vp]
        L.qkv_quantize_chunks.argtypes = [i32, P(P(qkv_config)), P(P(qkv_tensor)), P(P(qkv_side)), P(vp), vp, sz, vp]
        L.qkv_quantize_chunks_workspace_bytes.argtypes = [P(qkv_config), i64, i32, P(sz)]
        L.qkv_quantize_chunk_noalloc.argtypes = [P(qkv_config), P(qkv_tensor), P(qkv_side), vp, vp]
        L.qkv_attend_fresh.argtypes = [P(qkv_config), P(qkv_config), P(qkv_tensor), P(vp), P(vp), P(i64), i32,
                                       P(qkv_tensor), P(qkv_tensor), i32, vp, ct.c_float, P(qkv_tensor), vp, vp, sz, vp]
        L.qkv_temporal_layout.argtypes = [P(qkv_tcfg), i64, i32, P(sz), P(sz)]
        L.qkv_temporal_state_bytes.argtypes = [P(qkv_tcfg), P(sz)]
        L.qkv_temporal_encode.argtypes = [P(qkv_tcfg), P(qkv_tensor), i64, vp, vp, vp]
        L.qkv_temporal_decode.argtypes = [P(qkv_tcfg), i64, i32, vp, vp, P(qkv_tensor), vp]
        L.qkv_timing_enable.argtypes = [i32]
        L.qkv_timing_read.argtypes = [i32, P(qkv_kernel_time), P(i32)]
        for name in EXPORTED[2:]:
            getattr(L, name).restype = ct.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != QKV_OK:
        raise QkvError(status, lib().qkv_last_error().decode(errors="replace"))


def _ptr(t):
    """Device address of a torch tensor (None -> NULL)."""
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ct.c_void_p(int(stream))


def tensor_desc(t, n_heads: int | None = None) -> qkv_tensor:
    """qkv_tensor of a torch tensor shaped [N, H, 128] (any strides with a
    contiguous last dimension) or [N, 128] (one head)."""
    import torch
    if t.dim() == 2:
        t = t.unsqueeze(1)
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected [N, H, 128] with a contiguous last dimension")
    dt = {torch.float32: QKV_F32, torch.bfloat16: QKV_BF16}[t.dtype]
    return qkv_tensor(t.data_ptr(), dt, 0, t.shape[0], t.stride(0), t.stride(1))


def qkv_version() -> int:
    return lib().qkv_version()


def qkv_last_error() -> str:
    return lib().qkv_last_error().decode(errors="replace")


def qkv_chunk_layout(cfg: Config, n_tokens: int) -> qkv_layout:
    out = qkv_layout()
    _check(lib().qkv_chunk_layout(ct.byref(cfg.c()), n_tokens, ct.byref(out)))
    return out


def qkv_workspace_bytes(cfg: Config, max_chunk_tokens: int, n_query: int = 0, n_chunks: int = 0) -> int:
    out = ct.c_size_t()
    _check(lib().qkv_workspace_bytes(ct.byref(cfg.c()), max_chunk_tokens, n_query, n_chunks, ct.byref(out)))
    return out.value


def qkv_quantize_chunk(cfg: Config, x, packed, workspace, w=None, perm=None, U=None, stream=None):
    side = qkv_side(_ptr(w), _ptr(perm), _ptr(U))
    _check(lib().qkv_quantize_chunk(ct.byref(cfg.c()), ct.byref(tensor_desc(x)), ct.byref(side),
                                    _ptr(packed), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))


def qkv_quantize_chunk_noalloc(cfg: Config, x, packed, w=None, perm=None, U=None, stream=None):
    side = qkv_side(_ptr(w), _ptr(perm), _ptr(U))
    _check(lib().qkv_quantize_chunk_noalloc(ct.byref(cfg.c()), ct.byref(tensor_desc(x)), ct.byref(side),
                                            _ptr(packed), _stream(stream)))


def qkv_dequantize(cfg: Config, n_tokens: int, packed, out, stream=None):
    _check(lib().qkv_dequantize(ct.byref(cfg.c()), n_tokens, _ptr(packed), ct.byref(tensor_desc(out)),
                                _stream(stream)))


def qkv_attend(k_cfg: Config, v_cfg: Config, q, k_chunks, v_chunks, chunk_tokens, out, workspace,
               U=None, causal: bool = False, softmax_scale: float = 0.0, logits=None, stream=None):
    n = len(k_chunks)
    kp = (ct.c_void_p * n)(*[c.data_ptr() for c in k_chunks])
    vp_ = (ct.c_void_p * n)(*[c.data_ptr() for c in v_chunks])
    nt = (ct.c_int64 * n)(*[int(x) for x in chunk_tokens])
    _check(lib().qkv_attend(ct.byref(k_cfg.c()), ct.byref(v_cfg.c()), ct.byref(tensor_desc(q)), kp, vp_, nt, n,
                            _ptr(U), 1 if causal else 0, float(softmax_scale), ct.byref(tensor_desc(out)),
                            _ptr(logits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream)))


def qkv_attend_fresh(k_cfg: Config, v_cfg: Config, q, k_chunks, v_chunks, chunk_tokens, k_fresh, v_fresh,
                     frame_tokens: int, out, workspace, U=None, softmax_scale: float = 0.0, logits=None, stream=None):
    n = len(k_chunks)
    m = max(n, 1)
    kp = (ct.c_void_p * m)(*[c.data_ptr() for c in k_chunks])
    vp_ = (ct.c_void_p * m)(*[c.data_ptr() for c in v_chunks])
    nt = (ct.c_int64 * m)(*[int(x) for x in chunk_tokens])
    _check(lib().qkv_attend_fresh(ct.byref(k_cfg.c()), ct.byref(v_cfg.c()), ct.byref(tensor_desc(q)), kp, vp_, nt, n,
                                  ct.byref(tensor_desc(k_fresh)), ct.byref(tensor_desc(v_fresh)), int(frame_tokens),
                                  _ptr(U), float(softmax_scale), ct.byref(tensor_desc(out)), _ptr(logits),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def qkv_psac_fit(q_hist, n_heads: int, rank: int, n_int4: int, workspace, U_out=None, w_out=None,
                 perm_out=None, stream=None, energy: bool = True):
    """Returns the per-head energy fractions (host floats), or None with energy=False
    (then no eigensolver runs when rank == 0)."""
    en = (ct.c_float * n_heads)() if energy else None
    _check(lib().qkv_psac_fit(ct.byref(tensor_desc(q_hist)), n_heads, rank, n_int4, _ptr(U_out), _ptr(w_out),
                              _ptr(perm_out), en, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return list(en) if energy else None


def qkv_quantize_chunks_workspace_bytes(cfg: Config, n_tokens: int, n: int) -> int:
    out = ct.c_size_t()
    _check(lib().qkv_quantize_chunks_workspace_bytes(ct.byref(cfg.c()), n_tokens, n, ct.byref(out)))
    return out.value


def qkv_quantize_chunks(cfgs, xs, packs, workspace, sides=None, stream=None):
    """Batch of write paths in one set of launches; sides: list of (w, perm, U) or None."""
    n = len(xs)
    cc = [c.c() for c in cfgs]
    tt = [tensor_desc(x) for x in xs]
    ss = [qkv_side(_ptr(s[0]), _ptr(s[1]), _ptr(s[2])) if s is not None else qkv_side(None, None, None)
          for s in (sides or [None] * n)]
    cp = (ct.POINTER(qkv_config) * n)(*[ct.pointer(c) for c in cc])
    tp = (ct.POINTER(qkv_tensor) * n)(*[ct.pointer(t) for t in tt])
    sp = (ct.POINTER(qkv_side) * n)(*[ct.pointer(s) for s in ss])
    pk = (ct.c_void_p * n)(*[p.data_ptr() for p in packs])
    _check(lib().qkv_quantize_chunks(n, cp, tp, sp, pk, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def qkv_kmeans_assign(cfg: Config, y, centroids, labels, workspace, w=None, stream=None):
    _check(lib().qkv_kmeans_assign(ct.byref(cfg.c()), ct.byref(tensor_desc(y)), _ptr(centroids), _ptr(w),
                                   _ptr(labels), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def qkv_kmeans_update(cfg: Config, y, labels, centroids, workspace, counts=None, stream=None):
    _check(lib().qkv_kmeans_update(ct.byref(cfg.c()), ct.byref(tensor_desc(y)), _ptr(labels), _ptr(centroids),
                                   _ptr(counts), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def qkv_quant_pack(cfg: Config, y, labels, centroids, packed, stage: int = 0, perm=None, y_next=None,
                   stream=None):
    _check(lib().qkv_quant_pack(ct.byref(cfg.c()), ct.byref(tensor_desc(y)), _ptr(labels), _ptr(centroids),
                                _ptr(perm), _ptr(packed), stage, _ptr(y_next), _stream(stream)))


def qkv_timing_enable(on: bool):
    _check(lib().qkv_timing_enable(1 if on else 0))


def qkv_timing_read() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded since qkv_timing_enable(True)."""
    n = ct.c_int32()
    _check(lib().qkv_timing_read(0, None, ct.byref(n)))
    buf = (qkv_kernel_time * max(1, n.value))()
    _check(lib().qkv_timing_read(n.value, buf, ct.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n.value)}


def qkv_temporal_layout(cfg: TConfig, frame0: int, n_frames: int):
    """(bytes, [frame byte offsets]) of a packed run of the temporally stable codec."""
    nb = ct.c_size_t()
    offs = (ct.c_size_t * max(1, n_frames))()
    _check(lib().qkv_temporal_layout(ct.byref(cfg.c()), frame0, n_frames, ct.byref(nb), offs))
    return nb.value, [offs[i] for i in range(n_frames)]


def qkv_temporal_state_bytes(cfg: TConfig) -> int:
    nb = ct.c_size_t()
    _check(lib().qkv_temporal_state_bytes(ct.byref(cfg.c()), ct.byref(nb)))
    return nb.value


def qkv_temporal_encode(cfg: TConfig, x, frame0: int, state, packed, stream=None):
    _check(lib().qkv_temporal_encode(ct.byref(cfg.c()), ct.byref(tensor_desc(x)), frame0, _ptr(state), _ptr(packed),
                                     _stream(stream)))


def qkv_temporal_decode(cfg: TConfig, frame0: int, n_frames: int, packed, anchor, out, stream=None):
    _check(lib().qkv_temporal_decode(ct.byref(cfg.c()), frame0, n_frames, _ptr(packed), _ptr(anchor),
                                     ct.byref(tensor_desc(out)), _stream(stream)))
