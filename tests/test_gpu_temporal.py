"""GPU parity of the practitioner blog's temporally stable 2-bit codec against the
oracle (oracle/temporal.py): every packed section of every frame (codes, zero
points, scales, outlier values and channels, anchor values) and the rebuilt
values, bit for bit, through runs of frames with the state carried between
calls."""
import numpy as np
import pytest

import video_model_kv_amd as qk
from video_model_kv_amd import synth
from oracle import temporal as tp
from oracle.numerics import bf16_rne

import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _a256(x):
    return (x + 255) // 256 * 256


def _sections(cfg, th):
    """Byte offsets of the sections of a coded frame (the layout in include/qkv.h)."""
    lo = _a256(th * 4 * cfg.bits * 4)
    scale = lo + _a256(th * 8)
    oval = scale + _a256(th * 8)
    oidx = oval + _a256(th * 8)
    return lo, scale, oval, oidx


def _f16bits(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def _pack_codes(q, bits):
    """q [..., 4, 32] -> u32 words [..., 4 * bits] in the documented order."""
    per = 32 // bits
    q = q.astype(np.uint32).reshape(q.shape[:-1] + (bits, per))
    sh = (bits * np.arange(per)).astype(np.uint32)
    return np.bitwise_or.reduce(q << sh, axis=-1).reshape(q.shape[:-3] + (4 * bits,))


def _check_run(name, cfg, packed, frame0, frames, heads, H):
    """Packed bytes of a run against the oracle's frames (all positions, the listed heads)."""
    P = cfg.frame_tokens
    th = P * H
    nb, offs = qk.qkv_temporal_layout(cfg, frame0, len(frames))
    raw = packed.cpu().numpy()
    lo_o, sc_o, ov_o, oi_o = _sections(cfg, th)
    for f, fr in enumerate(frames):
        base = offs[f]
        if fr.anchor:
            got = raw[base: base + th * 256].view(np.uint16).reshape(P, H, 128)
            assert np.array_equal(got[:, heads], _f16bits(fr.values16)), f"{name} frame {frame0 + f}: anchor values"
            continue
        b = fr.blocks
        codes = raw[base: base + th * 16 * cfg.bits].view(np.uint32).reshape(P, H, 4 * cfg.bits)
        assert np.array_equal(codes[:, heads], _pack_codes(b.q, cfg.bits)), f"{name} frame {frame0 + f}: codes"
        for off, exp, what in ((lo_o, _f16bits(b.lo), "zero points"), (sc_o, _f16bits(b.scale), "scales"),
                               (ov_o, _f16bits(b.out_val), "outlier values")):
            got = raw[base + off: base + off + th * 8].view(np.uint16).reshape(P, H, 4)
            assert np.array_equal(got[:, heads], exp), f"{name} frame {frame0 + f}: {what}"
        got = raw[base + oi_o: base + oi_o + th * 4].reshape(P, H, 4)
        assert np.array_equal(got[:, heads], b.out_idx), f"{name} frame {frame0 + f}: outlier channels"


def _stream(name, x, cfg, runs, heads=None, f32=False, check_decode=True):
    """Code x [F, P, H, 128] in runs [(frame0, n)] on the device (state carried)
    and by the oracle (one call per run too), compare packed bytes and the
    rebuilt values of every run."""
    t = G.torch()
    F, P, H, _ = x.shape
    heads = list(range(H)) if heads is None else heads
    state = t.empty(qk.qkv_temporal_state_bytes(cfg), dtype=t.uint8, device=G.dev())
    ostate = None
    for frame0, n in runs:
        G.log(f"temporal {name}: frames {frame0}..{frame0 + n - 1} (P={P}, H={H}, bits={cfg.bits}, "
              f"anchor every {cfg.anchor_every}, decay {cfg.decay})")
        nb, _ = qk.qkv_temporal_layout(cfg, frame0, n)
        packed = t.zeros(nb, dtype=t.uint8, device=G.dev())
        anchor_before = state[P * H * 128 * 4:].clone()
        xd = G.to_dev(x[frame0:frame0 + n].reshape(n * P, H, 128), "f32" if f32 else "bf16")
        qk.qkv_temporal_encode(cfg, xd, frame0, state, packed)
        frames, ostate = tp.encode(x[frame0:frame0 + n][:, :, heads], frame0, ostate, bits=cfg.bits,
                                   anchor_every=cfg.anchor_every, decay=cfg.decay)
        _check_run(name, cfg, packed, frame0, frames, heads, H)
        if check_decode:
            for dt in ("f32", "bf16"):
                out = t.empty((n * P, H, 128), dtype=t.float32 if dt == "f32" else t.bfloat16, device=G.dev())
                qk.qkv_temporal_decode(cfg, frame0, n, packed, anchor_before, out)
                if dt == "f32":
                    got = out.cpu().numpy().reshape(n, P, H, 128)[:, :, heads]
                    exp = np.stack([fr.kv_hat for fr in frames])
                    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), f"{name}: rebuilt values"
                else:
                    got = out.view(t.int16).cpu().numpy().view(np.uint16).reshape(n, P, H, 128)[:, :, heads]
                    exp = G.f32_bits_to_bf16(bf16_rne(np.stack([fr.kv_hat for fr in frames])))
                    assert np.array_equal(got, exp), f"{name}: rebuilt bf16 values"
    # the state after the last run: feedback and anchor
    st = state.cpu().numpy()
    fb = st[: P * H * 128 * 4].view(np.float32).reshape(P, H, 128)[:, heads]
    an = st[P * H * 128 * 4:].view(np.uint16).reshape(P, H, 128)[:, heads]
    assert np.array_equal(fb.view(np.uint32), ostate.feedback.view(np.uint32)), f"{name}: feedback state"
    assert np.array_equal(an, _f16bits(ostate.anchor)), f"{name}: anchor state"


def _video(rng, nf, p, h, outliers=0.03):
    base = rng.standard_normal((p, h, 128)) * 3
    drift = rng.standard_normal((p, h, 128)) * 0.05
    x = np.stack([base + t * drift + rng.standard_normal((p, h, 128)) * 0.02 for t in range(nf)])
    x[..., 5] += 40 * (rng.random((nf, p, h)) < outliers)
    x[..., 77] -= 300 * (rng.random((nf, p, h)) < outliers)
    return bf16_rne(x).astype(np.float32)


def test_stream_in_runs_with_state():
    rng = np.random.default_rng(11)
    x = _video(rng, 12, 48, 2)
    cfg = qk.TConfig(n_heads=2, frame_tokens=48, bits=2, anchor_every=8, decay=0.8)
    _stream("runs", x, cfg, [(0, 4), (4, 4), (8, 4)])


def test_run_starting_mid_group_with_an_anchor_inside():
    """Frames 0-5, then a run 6..9 whose frame 8 is an anchor: frames 6-7 use
    the caller's anchor at decode, frames 9 the run's own."""
    rng = np.random.default_rng(12)
    x = _video(rng, 10, 40, 3)
    cfg = qk.TConfig(n_heads=3, frame_tokens=40, bits=2, anchor_every=8, decay=0.8)
    _stream("mid-group", x, cfg, [(0, 6), (6, 4)])


def test_fp32_input_four_bits_and_no_feedback():
    rng = np.random.default_rng(13)
    x = _video(rng, 9, 33, 2)
    x = (x * np.float32(1.0 + 2.0 ** -12)).astype(np.float32)     # off the bf16 grid
    _stream("f32-4bit", x, qk.TConfig(n_heads=2, frame_tokens=33, bits=4, anchor_every=5, decay=0.8),
            [(0, 3), (3, 6)], f32=True)
    _stream("decay0", x, qk.TConfig(n_heads=2, frame_tokens=33, bits=2, anchor_every=32, decay=0.0),
            [(0, 9)], f32=True)


def test_edge_blocks():
    """Blocks of equal values (scale 0), tied largest magnitudes (no outlier),
    opposite-signed tied magnitudes, all-zero blocks and lone large values."""
    rng = np.random.default_rng(14)
    P, H, nf = 16, 2, 6
    x = np.zeros((nf, P, H, 128), np.float32)
    x[:, 0] = 1.5                                      # constant blocks
    x[:, 1, :, 3] = x[:, 1, :, 9] = 7.0                # tied largest magnitudes
    x[:, 2, :, 4], x[:, 2, :, 20] = -9.0, 9.0          # tied, opposite signs
    x[:, 3] = bf16_rne(rng.standard_normal((nf, H, 128)))
    x[:, 3, :, 64] = 1000.0                            # one large value
    x[:, 4:] = bf16_rne(rng.standard_normal((nf, P - 4, H, 128)) * 0.5)
    x[1:, 5] = x[:1, 5]                                # static positions
    cfg = qk.TConfig(n_heads=H, frame_tokens=P, bits=2, anchor_every=4, decay=0.8)
    _stream("edges", x.astype(np.float32), cfg, [(0, 3), (3, 3)])


def test_full_size_one_minute_cache_sampled_heads():
    """The one-minute cache's keys, frames 0-39 (10 chunks of 4 frames, 1,560
    positions, 32 heads; an anchor at 0 and at 32) coded chunk by chunk; heads 0
    and 23 against the oracle, every section and the rebuilt values."""
    wl = synth.workload(5)
    P, H = wl.tokens_per_frame, wl.n_heads
    chunks = [synth.kv_chunk(wl, "K", c) for c in range(10)]
    x = np.concatenate(chunks).reshape(40, P, H, 128)
    cfg = qk.TConfig(n_heads=H, frame_tokens=P, bits=2, anchor_every=32, decay=0.8)
    _stream("minute-K", x, cfg, [(4 * c, 4) for c in range(10)], heads=[0, 23])
