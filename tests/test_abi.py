"""The C-ABI library: it loads, exports every entry point the header declares,
reports the documented layout, and rejects invalid arguments on the host before
touching a device (no GPU needed)."""
import ctypes as ct
import os
import re

import numpy as np
import pytest

from video_model_kv_amd import _binding as B
from oracle import quant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000            # an aligned address that validation never dereferences


def _declared():
    src = open(os.path.join(ROOT, "include", "qkv.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(qkv_[a-z_0-9]+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(B.EXPORTED)
    assert B.qkv_version() == 1


@pytest.mark.parametrize("bits,group,n4", [(2, 32, 0), (2, 64, 0), (4, 32, 0), (2, 16, 0), (2, 32, 26), (2, 128, 0)])
def test_layout_matches_independent_format(bits, group, n4):
    cfg = B.Config(n_heads=3, n_clusters=64, bits=bits, group=group, n_int4_channels=n4, n_stages=2, psac_rank=8)
    n = 1000
    L = B.qkv_chunk_layout(cfg, n)
    perm = np.arange(128)
    ref = quant.channel_layout(128, bits, group, n4, perm)
    assert L.words_per_token == ref.words
    assert L.groups_per_token == len(ref.groups)
    if n4:
        assert L.int4_words == ref.class_word0[1]
    al = lambda x: (x + 255) // 256 * 256
    assert L.stage_bytes_codes == al(3 * n * ref.words * 4)
    assert L.stage_bytes_scales == al(3 * n * len(ref.groups) * 2)
    assert L.stage_bytes_labels == al(3 * n)
    assert L.stage_bytes_centroids == al(3 * 64 * 128 * 2)
    offs = [L.off_codes, L.off_scales, L.off_labels, L.off_centroids, L.off_perm, L.off_psac]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.off_scales == L.off_codes + 2 * L.stage_bytes_codes
    assert L.bytes == L.off_psac + al(3 * n * 8 * 2)


def _cfg(**kw):
    base = dict(n_heads=2, n_clusters=16)
    base.update(kw)
    return B.Config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), B.QKV_EUNSUPPORTED),
    (dict(n_clusters=0), B.QKV_EINVAL),
    (dict(n_clusters=257), B.QKV_EINVAL),
    (dict(bits=3), B.QKV_EINVAL),
    (dict(group=24), B.QKV_EINVAL),
    (dict(group=8), B.QKV_EINVAL),
    (dict(n_stages=0), B.QKV_EINVAL),
    (dict(n_stages=5), B.QKV_EINVAL),
    (dict(psac_rank=9), B.QKV_EINVAL),
    (dict(n_int4_channels=128), B.QKV_EINVAL),
    (dict(n_int4_channels=10, bits=4), B.QKV_EINVAL),
    (dict(kmeans_iters=0), B.QKV_EINVAL),
    (dict(flags=4), B.QKV_EINVAL),
])
def test_invalid_configs(kw, status):
    with pytest.raises(B.QkvError) as e:
        B.qkv_chunk_layout(_cfg(**kw), 100)
    assert e.value.status == status
    assert len(B.qkv_last_error()) > 0


def test_too_few_tokens():
    with pytest.raises(B.QkvError) as e:
        B.qkv_chunk_layout(_cfg(), 15)
    assert e.value.status == B.QKV_EINVAL


def _tensor(n=100, dtype=B.QKV_BF16, ptr=FAKE, st=256, sh=128):
    return B.qkv_tensor(ptr, dtype, 0, n, st, sh)


def _quantize(cfg, x, side=None, packed=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lib = B.lib()
    side = side or B.qkv_side(None, None, None)
    return lib.qkv_quantize_chunk(ct.byref(cfg.c()), ct.byref(x), ct.byref(side), packed, ws, ws_bytes, None)


def test_quantize_validation_paths():
    cfg = _cfg()
    assert _quantize(cfg, _tensor(ptr=0)) == B.QKV_EINVAL                  # NULL data
    assert _quantize(cfg, _tensor(ptr=FAKE + 4)) == B.QKV_EINVAL           # misaligned
    assert _quantize(cfg, _tensor(dtype=7)) == B.QKV_EINVAL
    assert _quantize(cfg, _tensor(st=100)) == B.QKV_EINVAL                 # stride not a multiple of 8
    assert _quantize(cfg, _tensor(sh=64)) == B.QKV_EINVAL                  # heads overlap
    assert _quantize(cfg, _tensor(n=10)) == B.QKV_EINVAL                   # N < C
    assert _quantize(cfg, _tensor(), packed=None) == B.QKV_EINVAL
    assert _quantize(cfg, _tensor(), ws=None) == B.QKV_EWORKSPACE
    assert _quantize(cfg, _tensor(), ws_bytes=1000) == B.QKV_EWORKSPACE
    assert _quantize(_cfg(use_qsac=1), _tensor()) == B.QKV_EINVAL          # missing w
    assert _quantize(_cfg(n_int4_channels=26), _tensor()) == B.QKV_EINVAL  # missing perm
    assert _quantize(_cfg(psac_rank=8), _tensor()) == B.QKV_EINVAL         # missing U
    assert "U" in B.qkv_last_error()


def _quantize_batch(cfgs, xs, sides=None, packs=None, ws=FAKE, ws_bytes=1 << 40, n=None):
    lib = B.lib()
    n = len(xs) if n is None else n
    m = max(len(xs), 1)
    cc = [c.c() for c in cfgs]
    cp = (ct.POINTER(B.qkv_config) * m)(*[ct.pointer(c) for c in cc])
    tp = (ct.POINTER(B.qkv_tensor) * m)(*[ct.pointer(x) for x in xs])
    sides = sides or [B.qkv_side(None, None, None)] * m
    sp = (ct.POINTER(B.qkv_side) * m)(*[ct.pointer(s) for s in sides])
    pk = (ct.c_void_p * m)(*(packs or [FAKE] * m))
    return lib.qkv_quantize_chunks(n, cp, tp, sp, pk, ws, ws_bytes, None)


def test_quantize_batch_validation_paths():
    k, v = _cfg(), _cfg(bits=4)                       # bits may differ within a batch
    assert _quantize_batch([k, v], [_tensor(), _tensor()], ws_bytes=1000) == B.QKV_EWORKSPACE
    assert _quantize_batch([k], [_tensor()], n=0) == B.QKV_EINVAL
    assert _quantize_batch([k] * 17, [_tensor()] * 17) == B.QKV_EINVAL          # more than 16 problems
    assert _quantize_batch([k, _cfg(n_clusters=32)], [_tensor(), _tensor()]) == B.QKV_EINVAL
    assert _quantize_batch([k, _cfg(kmeans_iters=3)], [_tensor(), _tensor()]) == B.QKV_EINVAL
    assert _quantize_batch([k, _cfg(n_stages=2)], [_tensor(), _tensor()]) == B.QKV_EINVAL
    assert _quantize_batch([k, v], [_tensor(), _tensor(n=120)]) == B.QKV_EINVAL   # token counts differ
    assert _quantize_batch([k, v], [_tensor(), _tensor(dtype=B.QKV_F32)]) == B.QKV_EINVAL
    assert _quantize_batch([k, v], [_tensor(), _tensor()], packs=[FAKE, None]) == B.QKV_EINVAL
    assert _quantize_batch([k, _cfg(use_qsac=1)], [_tensor(), _tensor()]) == B.QKV_EINVAL   # missing w
    assert "problem 1" in B.qkv_last_error()
    one = B.qkv_quantize_chunks_workspace_bytes(k, 6240, 1)
    assert B.qkv_quantize_chunks_workspace_bytes(k, 6240, 12) == 12 * one
    assert one >= B.qkv_workspace_bytes(k, 6240) - 256
    with pytest.raises(B.QkvError):
        B.qkv_quantize_chunks_workspace_bytes(k, 6240, 17)


def test_workspace_sizes_grow_with_work():
    cfg = _cfg(n_heads=32, n_clusters=256)
    a = B.qkv_workspace_bytes(cfg, 6240)
    b = B.qkv_workspace_bytes(_cfg(n_heads=32, n_clusters=256, n_stages=3), 6240)
    c = B.qkv_workspace_bytes(cfg, 6240, 1560, 6)
    assert 0 < a < b and a <= c
    # centroids f32 + planes + norms at minimum
    assert a >= 32 * 256 * 128 * 4 + 32 * 2 * 256 * 128 * 2


def test_attend_validation_paths():
    lib = B.lib()
    cfg = _cfg()
    q = _tensor(n=64)
    out = B.qkv_tensor(FAKE, B.QKV_F32, 0, 64, 256, 128)
    chunks = (ct.c_void_p * 1)(FAKE)
    ntok = (ct.c_int64 * 1)(100)

    def call(k_cfg=cfg, v_cfg=cfg, q=q, out=out, n=1, ntok=ntok, U=None, causal=0, scale=0.0, ws_bytes=1 << 40):
        return lib.qkv_attend(ct.byref(k_cfg.c()), ct.byref(v_cfg.c()), ct.byref(q), chunks, chunks, ntok, n,
                              U, causal, scale, ct.byref(out), None, FAKE, ws_bytes, None)

    assert call(n=0) == B.QKV_EINVAL
    assert call(n=2000) == B.QKV_EINVAL
    assert call(k_cfg=_cfg(n_heads=3)) == B.QKV_EINVAL
    assert call(k_cfg=_cfg(psac_rank=8)) == B.QKV_EINVAL                  # no U
    assert call(v_cfg=_cfg(psac_rank=8)) == B.QKV_EINVAL                  # PSAC on V
    assert call(out=B.qkv_tensor(FAKE, B.QKV_BF16, 0, 64, 256, 128)) == B.QKV_EINVAL
    assert call(ntok=(ct.c_int64 * 1)(5)) == B.QKV_EINVAL                 # chunk smaller than C
    assert call(causal=1) == B.QKV_EINVAL                                 # Nq != Nk
    assert call(scale=-1.0) == B.QKV_EINVAL
    assert call(ws_bytes=16) == B.QKV_EWORKSPACE


def test_psac_fit_validation_paths():
    lib = B.lib()
    q = _tensor(n=4096)
    f = ct.c_float * 2
    assert lib.qkv_psac_fit(ct.byref(q), 2, 9, 0, FAKE, None, None, f(), FAKE, 1 << 40, None) == B.QKV_EINVAL
    assert lib.qkv_psac_fit(ct.byref(q), 2, 8, 0, None, None, None, f(), FAKE, 1 << 40, None) == B.QKV_EINVAL
    assert lib.qkv_psac_fit(ct.byref(q), 0, 8, 0, FAKE, None, None, f(), FAKE, 1 << 40, None) == B.QKV_EINVAL
    assert lib.qkv_psac_fit(ct.byref(q), 2, 8, 0, FAKE, None, None, f(), FAKE, 64, None) == B.QKV_EWORKSPACE


def test_kernel_timing_switch_without_a_gpu():
    """The timing record is host state: switching it on and reading an empty
    record needs no device; a NULL count pointer is rejected."""
    B.qkv_timing_enable(True)
    assert B.qkv_timing_read() == {}
    B.qkv_timing_enable(False)
    assert B.lib().qkv_timing_read(0, None, None) == B.QKV_EINVAL


def test_temporal_layout_arithmetic():
    """Anchor frames hold fp16 values; the others codes, zero points, scales,
    outlier values and channels, each section 256-byte aligned."""
    def a256(x):
        return (x + 255) // 256 * 256
    cfg = B.TConfig(n_heads=3, frame_tokens=50, bits=2, anchor_every=4)
    th = 150
    coded = a256(th * 4 * 2 * 4) + 3 * a256(th * 4 * 2) + a256(th * 4)
    anchor = a256(th * 128 * 2)
    nb, offs = B.qkv_temporal_layout(cfg, 2, 5)            # frames 2, 3, [4 anchor], 5, 6
    assert offs == [0, coded, 2 * coded, 2 * coded + anchor, 3 * coded + anchor]
    assert nb == 4 * coded + anchor
    assert B.qkv_temporal_state_bytes(cfg) == th * 128 * 6


@pytest.mark.parametrize("kw,frame0,n", [
    (dict(bits=3), 0, 4), (dict(decay=1.5), 0, 4), (dict(decay=-0.1), 0, 4), (dict(anchor_every=0), 0, 4),
    (dict(n_heads=0), 0, 4), (dict(frame_tokens=0), 0, 4), ({}, -1, 4), ({}, 0, 0), ({}, 0, 65),
])
def test_temporal_invalid_arguments(kw, frame0, n):
    cfg = B.TConfig(**dict(dict(n_heads=2, frame_tokens=8), **kw))
    with pytest.raises(B.QkvError) as e:
        B.qkv_temporal_layout(cfg, frame0, n)
    assert e.value.status == B.QKV_EINVAL
