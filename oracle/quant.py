"""Per-group symmetric quantizer, channel classes and bit packing (oracle; test
infrastructure only).

Scale and rounding: QVG notes, section "Research background / core tension":
S = max|X| / (2^(b-1) - 1) over a group and X_INT = round(X / S); the reading
taken stores S in bf16 and quantizes with the stored S.  Groups run along the
channels of one token (2-bit trap explainer, section two, its demo groups a
token's channels in fixed-size runs).  The clamp range [-2^(b-1), 2^(b-1) - 1]
is the signed b-bit range (same demo).  Ties round to even.  S == 0 gives q = 0.

Dequantization: QVG notes, "Method / Overall framework": x_hat = S * q + C_i.

Mixed precision: 2-bit trap explainer, section five (advice one), and the
practitioner blog, section 3.2: the channels a table marks sensitive get 4 bits,
the rest 2 bits.  Channels are listed in ``perm`` order: the 4-bit class first,
then the 2-bit class; each class is cut into runs of ``group`` channels (the
last run may be shorter) and starts on a 32-bit word boundary in the packed
codes.

Packed code format (the library's documented layout, restated independently):
stored code u = q + 2^(b-1); in a class, the channel at class position p of a
b-bit class sits in word (class_word0 + p // (32 / b)) at bit b * (p % (32 / b)),
little-endian within a uint32.

Pins (tests/test_oracle_quant.py): scale formula on hand-worked groups, the
|r - S q| <= S/2 bound, the zero-centroid case against a separate textbook
per-group quantizer, and a pack/unpack round trip with single-bit placement.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import bf16_rne


@dataclass(frozen=True)
class Group:
    channels: np.ndarray   # original channel indices, in perm order
    bits: int


@dataclass(frozen=True)
class ChannelLayout:
    head_dim: int
    perm: np.ndarray        # int64 [d], class order
    classes: tuple          # ((n_channels, bits), ...)
    groups: tuple           # (Group, ...) in storage order
    class_word0: tuple      # first word of each class
    words: int              # u32 words per token
    # per channel (original index): class id, position in class, bits
    ch_class: np.ndarray
    ch_pos: np.ndarray
    ch_bits: np.ndarray


def channel_layout(head_dim: int, bits: int, group: int, n_int4: int = 0, perm=None) -> ChannelLayout:
    """Channel classes, groups and word offsets of one token-head."""
    d = head_dim
    if perm is None:
        perm = np.arange(d)
    perm = np.asarray(perm, dtype=np.int64)
    if sorted(perm.tolist()) != list(range(d)):
        raise ValueError("perm must be a permutation of the channels")
    if n_int4 > 0:
        classes = ((n_int4, 4), (d - n_int4, 2))
    else:
        classes = ((d, bits),)
    groups, word0 = [], []
    ch_class = np.zeros(d, np.int64)
    ch_pos = np.zeros(d, np.int64)
    ch_bits = np.zeros(d, np.int64)
    start, w = 0, 0
    for ci, (n_c, b) in enumerate(classes):
        chans = perm[start:start + n_c]
        word0.append(w)
        for p, ch in enumerate(chans):
            ch_class[ch], ch_pos[ch], ch_bits[ch] = ci, p, b
        for g0 in range(0, n_c, group):
            groups.append(Group(channels=chans[g0:g0 + group], bits=b))
        w += -(-n_c * b // 32)
        start += n_c
    return ChannelLayout(d, perm, classes, tuple(groups), tuple(word0), w, ch_class, ch_pos, ch_bits)


def scale_of(amax: np.ndarray, bits: int) -> np.ndarray:
    """Stored scale: bf16(fp32(amax / (2^(b-1) - 1)))."""
    qmax = np.float32(2 ** (bits - 1) - 1)
    s32 = (np.asarray(amax, np.float32) / qmax).astype(np.float32)
    return bf16_rne(s32)


def quantize_groups(r: np.ndarray, layout: ChannelLayout):
    """Quantize residuals r (float32 [N, d]) group by group.

    Returns q (int8 [N, d], original channel order) and the stored scales
    (float32, bf16-exact, [N, n_groups]) in storage order.
    """
    r = np.asarray(r, dtype=np.float32)
    n = r.shape[0]
    q = np.zeros(r.shape, dtype=np.int8)
    scales = np.zeros((n, len(layout.groups)), dtype=np.float32)
    for gi, g in enumerate(layout.groups):
        block = r[:, g.channels]
        amax = np.abs(block).max(axis=1)
        s = scale_of(amax, g.bits)
        scales[:, gi] = s
        lo, hi = -(2 ** (g.bits - 1)), 2 ** (g.bits - 1) - 1
        safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        ratio = (block / safe[:, None]).astype(np.float32)
        qq = np.clip(np.rint(ratio), lo, hi)
        qq[s == 0] = 0
        q[:, g.channels] = qq.astype(np.int8)
    return q, scales


def expand_scales(scales: np.ndarray, layout: ChannelLayout) -> np.ndarray:
    """Per-channel scale (float32 [N, d], original channel order)."""
    out = np.zeros((scales.shape[0], layout.head_dim), np.float32)
    for gi, g in enumerate(layout.groups):
        out[:, g.channels] = scales[:, gi:gi + 1]
    return out


def dequantize(q: np.ndarray, scales: np.ndarray, c_rows: np.ndarray, layout: ChannelLayout) -> np.ndarray:
    """x_hat = fp32(S * q + C) with C the token's bf16 centroid row (float32 values)."""
    sq = (expand_scales(scales, layout) * q.astype(np.float32)).astype(np.float32)
    return (sq + np.asarray(c_rows, np.float32)).astype(np.float32)


def pack_codes(q: np.ndarray, layout: ChannelLayout) -> np.ndarray:
    """uint32 [N, words]: u = q + 2^(b-1) at the documented bit position."""
    n = q.shape[0]
    words = np.zeros((n, layout.words), dtype=np.uint64)
    for ch in range(layout.head_dim):
        b = int(layout.ch_bits[ch])
        per = 32 // b
        p = int(layout.ch_pos[ch])
        wi = layout.class_word0[int(layout.ch_class[ch])] + p // per
        shift = b * (p % per)
        u = (q[:, ch].astype(np.int64) + 2 ** (b - 1)).astype(np.uint64)
        if np.any(u >= 2 ** b):
            raise ValueError("code out of range")
        words[:, wi] |= u << np.uint64(shift)
    return words.astype(np.uint32)


def unpack_codes(words: np.ndarray, layout: ChannelLayout) -> np.ndarray:
    """Inverse of pack_codes: int8 q [N, d] in original channel order."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    q = np.zeros((words.shape[0], layout.head_dim), np.int8)
    for ch in range(layout.head_dim):
        b = int(layout.ch_bits[ch])
        per = 32 // b
        p = int(layout.ch_pos[ch])
        wi = layout.class_word0[int(layout.ch_class[ch])] + p // per
        u = (words[:, wi] >> np.uint64(b * (p % per))) & np.uint64(2 ** b - 1)
        q[:, ch] = (u.astype(np.int64) - 2 ** (b - 1)).astype(np.int8)
    return q
