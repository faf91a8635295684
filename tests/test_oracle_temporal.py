"""Pins of the practitioner blog's temporally stable 2-bit scheme (oracle)."""
import numpy as np
import pytest

from oracle import temporal as tp


def test_outlier_rule_is_the_p99_of_the_block():
    """Values above numpy's P99 (linear interpolation) of a block's magnitudes:
    the unique largest one, or none when the two largest tie."""
    rng = np.random.default_rng(1)
    r = (rng.standard_normal((2000, 32)) * rng.uniform(0.1, 50, (2000, 1))).astype(np.float32)
    r[::7, 3] = r[::7, 9]                       # some top-two ties (when these are the largest)
    r[::11, 5] = -np.abs(r[::11]).max(axis=1)   # equal magnitudes of opposite sign
    r[::11, 6] = np.abs(r[::11]).max(axis=1)
    p99 = np.percentile(np.abs(r).astype(np.float64), 99, axis=1, keepdims=True)
    assert np.array_equal(tp.outlier_mask(r), np.abs(r) > p99)


def test_hand_worked_block():
    """r = [1, -0.5, 3, 0.25], 2 bits: 3 is the outlier; lo = -0.5, S = 1.5/3 = 0.5;
    q = rint([3, 0, -, 1.5]) = [3, 0, 0, 2] (half to even); r_hat = [1, -0.5, 3, 0.5]."""
    b = tp.quantize_blocks(np.array([1.0, -0.5, 3.0, 0.25], np.float32), 2, 4)
    assert b.out_idx.tolist() == [2] and b.out_val.tolist() == [3.0]
    assert b.lo.tolist() == [-0.5] and b.scale.tolist() == [0.5]
    assert b.q.tolist() == [[3, 0, 0, 2]]
    assert b.r_hat.tolist() == [1.0, -0.5, 3.0, 0.5]


def test_quantizer_bound():
    """|r - r_hat| <= S/2 + |min - lo| on the non-outlier values (fp16 rounding of
    the zero point); outliers rebuild as their fp16 value."""
    rng = np.random.default_rng(2)
    r = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 100, (500, 1))).astype(np.float32)
    b = tp.quantize_blocks(r, 2, 32)
    rb, hb = r.reshape(500, 4, 32), b.r_hat.reshape(500, 4, 32)
    out = tp.outlier_mask(rb)
    inner_min = np.where(out, np.inf, rb).min(axis=-1)
    slack = b.scale / 2 * (1 + 1e-6) + np.abs(inner_min - b.lo) + 1e-6 * np.abs(rb).max(axis=-1)
    assert np.all(np.where(out, 0, np.abs(rb - hb)) <= slack[..., None])
    assert np.array_equal(hb[out], r.reshape(500, 4, 32)[out].astype(np.float16).astype(np.float32))


def _video(rng, nf, p=48, h=2, d=64):
    base = rng.standard_normal((p, h, d)) * 3
    drift = rng.standard_normal((p, h, d)) * 0.05
    x = np.stack([base + t * drift + rng.standard_normal((p, h, d)) * 0.02 for t in range(nf)])
    x[..., 5] += 40 * (rng.random((nf, p, h)) < 0.03)       # sparse large values
    return x.astype(np.float32).astype(np.float16).astype(np.float32)


def test_error_feedback_delta_sigma_invariant():
    """The quantizer sees kv_t + 0.8 e_{t-1} (e = kv - kv_hat), so its own error
    is e_t + 0.8 e_{t-1}: on non-outlier values it stays within S_t/2 + |min -
    lo| (the zero point's fp16 rounding), frame after frame, across an anchor at
    frame 32, where the stream rebuilds fp16(kv) and the loop restarts."""
    rng = np.random.default_rng(3)
    kv = _video(rng, 40)
    frames, _ = tp.encode(kv, 0, None, group=32)
    checked = 0
    for t in range(1, 40):
        fr = frames[t]
        if fr.anchor:
            assert t % 32 == 0
            assert np.array_equal(fr.kv_hat, kv[t].astype(np.float16).astype(np.float32))
            continue
        e_prev = (kv[t - 1] - frames[t - 1].kv_hat).astype(np.float32)
        anchor = frames[t - t % 32].kv_hat
        r = ((kv[t] + np.float32(0.8) * e_prev).astype(np.float32) - anchor).astype(np.float32)
        rb = r.reshape(r.shape[:-1] + (2, 32))
        out = tp.outlier_mask(rb)
        inner_min = np.where(out, np.inf, rb).min(axis=-1)
        b = fr.blocks
        slack = 1e-6 * (np.abs(rb).max(axis=-1) + np.abs(anchor).reshape(rb.shape).max(axis=-1))
        bound = b.scale / 2 + np.abs(inner_min - b.lo) + slack
        qerr = (kv[t].astype(np.float64) - fr.kv_hat + 0.8 * e_prev.astype(np.float64)).reshape(rb.shape)
        assert np.all(np.where(out, 0, np.abs(qerr)) <= bound[..., None])
        checked += 1
    assert checked == 38


def test_decay_zero_is_independent_per_frame_quantization():
    rng = np.random.default_rng(4)
    kv = _video(rng, 6)
    frames, _ = tp.encode(kv, 0, None, decay=0.0, group=32)
    anchor = frames[0].kv_hat
    for t in range(1, 6):
        ref = (anchor + tp.quantize_blocks((kv[t] - anchor).astype(np.float32), 2, 32).r_hat).astype(np.float32)
        assert np.array_equal(frames[t].kv_hat, ref)


def test_anchor_only_stream_and_static_video():
    rng = np.random.default_rng(5)
    kv = _video(rng, 5)
    frames, _ = tp.encode(kv, 0, None, anchor_every=1)
    for t in range(5):
        assert np.array_equal(frames[t].kv_hat, kv[t].astype(np.float16).astype(np.float32))
    static = np.repeat(kv[:1], 7, axis=0)             # fp16-exact, identical frames
    frames, st = tp.encode(static, 0, None)
    for fr in frames:
        assert np.array_equal(fr.kv_hat, static[0])
    assert not np.any(st.feedback)


def test_chunked_stream_equals_one_call():
    """The state carries feedback and anchor: 3 chunks of 4 frames (frames 30-41,
    an anchor at 32) equal one call over the 12 frames."""
    rng = np.random.default_rng(6)
    kv = _video(rng, 14)
    _, st0 = tp.encode(kv[:2], 28, None, anchor_every=28)    # a stream that starts at an anchor
    whole, _ = tp.encode(kv[2:], 30, st0, anchor_every=28)
    st = st0
    parts = []
    for c in range(3):
        fr, st = tp.encode(kv[2 + 4 * c: 6 + 4 * c], 30 + 4 * c, st, anchor_every=28)
        parts += fr
    for a, b in zip(whole, parts):
        assert np.array_equal(a.kv_hat, b.kv_hat)
