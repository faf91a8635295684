"""Temporally stable 2-bit KV compression of the practitioner blog (oracle; test
infrastructure only).

Practitioner blog, sections 3.3-3.5 (and 3.6 for the chain):
  * outlier separation (section 3.4): in every quantization block, values whose
    magnitude exceeds the block's P99 are kept aside in fp16;
  * dynamic clipping (section 3.4): the block's own minimum and maximum set an
    asymmetric scale and zero point, stored with the block;
  * temporal anchors (section 3.3): frames are grouped by 32; the group's first
    frame is kept in fp16, and every other frame quantizes its residual against
    the group's prediction;
  * error feedback (section 3.5): the error of frame t, measured against the
    original (uncompensated) values, is decayed by 0.8 and added to frame t+1
    before it is quantized -- a first-order delta-sigma loop, serial over frames.

Readings taken where the page is silent or its pseudo-code lost its operators:
  * a block is one token-head's run of ``group`` consecutive channels (32), the
    grouping of the quantizer of the QVG notes;
  * P99 by linear interpolation over the block's magnitudes: for blocks of at
    most 100 values it lies strictly between the two largest magnitudes when they
    differ, so the outlier is the block's largest-magnitude value when that
    magnitude is unique (first index), none otherwise -- at most one per block;
  * the remaining values quantize as q = clamp(rint((r - lo) / S), 0, 2^b - 1)
    with lo = fp16(min), S = fp16((max - lo) / (2^b - 1)) (S <= 0: q = 0), and
    rebuild as lo + q S; the outlier rebuilds as its fp16 value;
  * the group's prediction is its anchor frame as stored (fp16), position by
    position (token i of frame t against token i of the anchor frame);
  * anchor frames store fp16(kv) uncompensated (the anchor resets the error, as
    the page says); the feedback after any frame is 0.8 (kv - kv_hat), the
    pseudo-code's "feedback = 0.8 * err" with err = kv_float - kv_dequant;
  * arithmetic in float32, every operation rounded once in the order written;
    fp16 conversions round to nearest even; inputs within the fp16 range.

Pins (tests/test_oracle_temporal.py): the outlier rule against numpy.percentile;
a hand-worked block; the quantizer's bound |r - r_hat| <= S/2 on non-outliers;
the delta-sigma invariant |e_t + 0.8 e_{t-1}| <= S_t/2; decay 0 reduces to
independent per-frame quantization; anchor-only streams rebuild fp16(kv); a
static fp16-exact video rebuilds exactly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32


def _f16(x) -> np.ndarray:
    """Round to fp16 (nearest even), back to float32."""
    return np.asarray(x, F32).astype(np.float16).astype(F32)


def outlier_mask(r: np.ndarray) -> np.ndarray:
    """[..., g] bool: the block's unique largest magnitude (first index), if any."""
    mag = np.abs(np.asarray(r, F32))
    s = np.sort(mag, axis=-1)
    unique = s[..., -1] > s[..., -2]
    first = np.argmax(mag, axis=-1)
    k = np.arange(mag.shape[-1])
    return unique[..., None] & (k == first[..., None])


@dataclass
class Blocks:
    q: np.ndarray         # uint8 [..., G, g] codes in [0, 2^b - 1] (0 at the outlier)
    lo: np.ndarray        # float32 (fp16 values) [..., G]
    scale: np.ndarray     # float32 (fp16 values) [..., G]
    out_idx: np.ndarray   # uint8 [..., G]: channel of the outlier in the block, 255 = none
    out_val: np.ndarray   # float32 (fp16 values) [..., G]; 0 when none
    r_hat: np.ndarray     # float32 [..., G, g] rebuilt values


def quantize_blocks(r: np.ndarray, bits: int, group: int) -> Blocks:
    """Outlier split + asymmetric min/max quantization of r [..., d] by blocks of
    ``group`` channels."""
    r = np.asarray(r, F32)
    d = r.shape[-1]
    rb = r.reshape(r.shape[:-1] + (d // group, group))
    out = outlier_mask(rb)
    inner_min = np.where(out, F32(np.inf), rb).min(axis=-1)
    inner_max = np.where(out, F32(-np.inf), rb).max(axis=-1)
    lo = _f16(inner_min)
    levels = F32(2 ** bits - 1)
    scale = _f16((inner_max - lo).astype(F32) / levels)
    pos = scale > 0
    s_safe = np.where(pos, scale, F32(1.0))[..., None]
    t = ((rb - lo[..., None]).astype(F32) / s_safe).astype(F32)
    q = np.where(pos[..., None], np.clip(np.rint(t), 0, 2 ** bits - 1), 0).astype(F32)
    q = np.where(out, F32(0), q)
    r_hat = (lo[..., None] + (q * scale[..., None]).astype(F32)).astype(F32)
    out_val16 = _f16(rb)
    r_hat = np.where(out, out_val16, r_hat)
    has = out.any(axis=-1)
    out_idx = np.where(has, np.argmax(out, axis=-1), 255).astype(np.uint8)
    out_val = np.where(out, out_val16, F32(0)).sum(axis=-1, dtype=F32).astype(F32)
    return Blocks(q.astype(np.uint8), lo, scale, out_idx, out_val, r_hat.reshape(r.shape))


@dataclass
class State:
    feedback: np.ndarray  # float32 [P, H, d]
    anchor: np.ndarray    # float32 (fp16 values) [P, H, d]: the current group's anchor as stored


@dataclass
class Frame:
    anchor: bool
    values16: np.ndarray | None   # anchor frames: float32 (fp16 values) [P, H, d]
    blocks: Blocks | None         # other frames: the quantized residual against the anchor
    kv_hat: np.ndarray            # float32 [P, H, d]


def encode(kv: np.ndarray, frame0: int, state: State | None, bits: int = 2, group: int = 32,
           anchor_every: int = 32, decay: float = 0.8):
    """Frames frame0 .. frame0 + F - 1 of kv [F, P, H, d] (float32, bf16 values),
    serially.  ``state`` carries the feedback and the anchor from the previous
    call (None before the first frame, which must then be an anchor frame).
    Returns (frames, new state)."""
    kv = np.asarray(kv, F32)
    nf = kv.shape[0]
    c = F32(decay)
    if state is None:
        if frame0 % anchor_every:
            raise ValueError("the first frame of a stream must be an anchor frame")
        state = State(np.zeros(kv.shape[1:], F32), np.zeros(kv.shape[1:], F32))
    fb, anchor = state.feedback.copy(), state.anchor.copy()
    frames = []
    for i in range(nf):
        x = kv[i]
        if (frame0 + i) % anchor_every == 0:
            a16 = _f16(x)
            anchor = a16
            kv_hat = a16
            frames.append(Frame(True, a16, None, kv_hat))
        else:
            comp = (x + fb).astype(F32)
            r = (comp - anchor).astype(F32)
            blk = quantize_blocks(r, bits, group)
            kv_hat = (anchor + blk.r_hat).astype(F32)
            frames.append(Frame(False, None, blk, kv_hat))
        fb = (c * (x - kv_hat).astype(F32)).astype(F32)
    return frames, State(fb, anchor)
