"""Seeded synthetic KV caches and queries shaped like the pages' workloads.

This module only draws inputs: it holds no step of the quantizer or of the
attention.  The library, its tests, the CPU oracle's tests and the benchmark
all take their inputs from here, so that both sides of every comparison see
the same bytes.

Workload shapes (QVG notes, "Research background / pain points": a 5 s 480p
clip is about 38K latent tokens; the reading taken is 24 latent frames of
30 x 52 = 1,560 tokens, 37,440 tokens, processed in chunks of 4 frames).  KV
statistics (QVG notes, "core tension"): max|K| is of order 1e2 and max|V| of
order 1e3, with outlier channels that change from token to token; tokens have
strong spatio-temporal redundancy ("angle of attack").

Recipe (NumPy PCG64; root seed 20261200 + config id; one child stream per
(head, tensor, role[, chunk]); values built in float64, rounded to float32 and,
for bf16 configs, to bfloat16 with round-to-nearest-even by torch):

* Tiny (config 1): 32 prototypes mu_p ~ N(0, I); each has 4 distinct outlier
  channels with random signs.  Token i picks p_i uniformly; y = mu_p +
  0.1 N(0, I); each outlier channel adds sign * U(50, 100) (K) or
  U(500, 1000) (V, from its own prototype set).  Queries N(0, I), float32.
* Field configs (2-5): per (head, tensor) 32 prototypes as above, placed as a
  spatially smooth field: a token's region is the nearest of 32 Voronoi seeds
  in the 30 x 52 plane, each seed drifting with a velocity U(-0.5, 0.5)
  tokens/frame per axis.  y = mu_region + phi + 0.1 N(0, I) + outliers of the
  region's prototype with per-token magnitude, where phi_k = 0.5 / sqrt(3) *
  sum_{m=1..3} cos(2 pi (kappa_m . (y, x) + omega_m f) + theta_km), with
  |kappa_m| <= 1/16 cycles/token and |omega_m| <= 1/24 cycles/frame.
  Queries N(0, I) bf16 (configs 2, 3).
* Query process of configs 4 and 5: q = B a with B a per-head random orthogonal
  matrix (QR of a Gaussian, signs fixed by diag(R) > 0), a_k ~ N(0, 20) for the
  first 8 coordinates and N(0, 1) for the rest; 4,096 history queries and
  1,560 attending queries, bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

ROOT_SEED = 20261200
FRAME_H, FRAME_W = 30, 52
TOKENS_PER_FRAME = FRAME_H * FRAME_W          # 1,560
N_PROTOTYPES = 32
N_OUTLIER_CH = 4
ROLE = {"proto": 0, "noise": 1, "outlier": 2, "field": 3, "query": 4, "hist": 5,
        "basis": 6, "label": 7}
TENSOR = {"K": 0, "V": 1, "Q": 2}


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    n_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    frames: int
    chunk_frames: int
    n_clusters: int
    n_stages: int
    bits: int
    group: int
    n_query: int
    causal: bool
    qsac: bool = False
    qsac_range: bool = False      # QSAC weights also take each stage's channel ranges (keys)
    psac_rank: int = 0
    n_int4: int = 0
    n_hist: int = 0
    kmeans_iters: int = 10
    tokens_per_frame: int = TOKENS_PER_FRAME

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def n_chunks(self) -> int:
        return -(-self.frames // self.chunk_frames)

    @property
    def n_tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    def chunk_range(self, c: int):
        t0 = c * self.chunk_tokens
        return t0, min(self.n_tokens, t0 + self.chunk_tokens)

    @property
    def seed(self) -> int:
        return ROOT_SEED + self.cid


WORKLOADS = {
    1: Workload(1, "tiny", 1, 128, "f32", 1, 1, 64, 1, 2, 64, 1560, True),
    2: Workload(2, "cache5s", 32, 128, "bf16", 24, 4, 256, 1, 2, 32, 1560, False),
    3: Workload(3, "progressive3", 32, 128, "bf16", 24, 4, 256, 3, 2, 32, 1560, False),
    4: Workload(4, "quantwm", 32, 128, "bf16", 24, 4, 256, 1, 2, 32, 1560, False,
                qsac=True, psac_rank=8, n_hist=4096),
    5: Workload(5, "minute", 32, 128, "bf16", 288, 4, 256, 1, 2, 32, 1560, False,
                n_int4=26, n_hist=4096),
}
# the QuantWM cache's data (same seed) with QSAC's residual-range factor
WORKLOADS[6] = replace(WORKLOADS[4], name="quantwm-range", qsac_range=True)


def workload(cid: int, **over) -> Workload:
    """The named workload, optionally shrunk (e.g. fewer heads or frames) for tests."""
    return replace(WORKLOADS[cid], **over)


def _rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def round_to(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 values exactly representable in the workload dtype."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).to(torch.float32).numpy()


def _prototypes(wl: Workload, head: int, tensor: str):
    r = _rng(wl.seed, head, TENSOR[tensor], ROLE["proto"])
    mu = r.standard_normal((N_PROTOTYPES, wl.head_dim))
    ch = np.stack([r.choice(wl.head_dim, N_OUTLIER_CH, replace=False) for _ in range(N_PROTOTYPES)])
    sign = r.choice(np.array([-1.0, 1.0]), size=(N_PROTOTYPES, N_OUTLIER_CH))
    return mu, ch, sign


def _outlier_range(tensor: str):
    return (50.0, 100.0) if tensor == "K" else (500.0, 1000.0)


def _tiny_tensor(wl: Workload, head: int, tensor: str, t0: int, t1: int) -> np.ndarray:
    mu, ch, sign = _prototypes(wl, head, tensor)
    n_all = wl.n_tokens
    p_all = _rng(wl.seed, head, TENSOR[tensor], ROLE["label"]).integers(0, N_PROTOTYPES, n_all)
    noise = _rng(wl.seed, head, TENSOR[tensor], ROLE["noise"]).standard_normal((n_all, wl.head_dim))
    lo, hi = _outlier_range(tensor)
    mag = _rng(wl.seed, head, TENSOR[tensor], ROLE["outlier"]).uniform(lo, hi, (n_all, N_OUTLIER_CH))
    p = p_all[t0:t1]
    y = mu[p] + 0.1 * noise[t0:t1]
    rows = np.arange(t1 - t0)[:, None]
    y[rows, ch[p]] += sign[p] * mag[t0:t1]
    return y


def _field_tensor(wl: Workload, head: int, tensor: str, t0: int, t1: int) -> np.ndarray:
    """Tokens t0..t1 (frame-major raster order) of one (head, tensor) field."""
    mu, ch, sign = _prototypes(wl, head, tensor)
    rf = _rng(wl.seed, head, TENSOR[tensor], ROLE["field"])
    seeds = np.stack([rf.uniform(0, FRAME_H, N_PROTOTYPES), rf.uniform(0, FRAME_W, N_PROTOTYPES)], 1)
    vel = rf.uniform(-0.5, 0.5, (N_PROTOTYPES, 2))
    kappa = rf.uniform(-1.0, 1.0, (3, 2)) * (1.0 / 16.0) / np.sqrt(2.0)
    omega = rf.uniform(-1.0, 1.0, 3) * (1.0 / 24.0)
    theta = rf.uniform(0.0, 2.0 * np.pi, (3, wl.head_dim))
    tok = np.arange(t0, t1)
    f = tok // wl.tokens_per_frame
    pos = tok % wl.tokens_per_frame
    yy = (pos // FRAME_W).astype(np.float64)
    xx = (pos % FRAME_W).astype(np.float64)
    # region: nearest drifting seed (ties -> lowest seed index via argmin)
    sy = seeds[None, :, 0] + vel[None, :, 0] * f[:, None]
    sx = seeds[None, :, 1] + vel[None, :, 1] * f[:, None]
    region = np.argmin((yy[:, None] - sy) ** 2 + (xx[:, None] - sx) ** 2, axis=1)
    # smooth field phi = [cos a_m, sin a_m] @ [cos theta; -sin theta] * 0.5 / sqrt(3)
    a = 2.0 * np.pi * (np.outer(yy, kappa[:, 0]) + np.outer(xx, kappa[:, 1]) + np.outer(f, omega))
    basis = np.concatenate([np.cos(a), np.sin(a)], 1)
    coef = np.concatenate([np.cos(theta), -np.sin(theta)], 0) * (0.5 / np.sqrt(3.0))
    phi = basis @ coef
    # per-chunk noise/magnitude streams, so any chunk is generated on its own
    y = mu[region] + phi
    lo, hi = _outlier_range(tensor)
    c0 = t0 // wl.chunk_tokens
    c1 = -(-t1 // wl.chunk_tokens)
    for c in range(c0, c1):
        a0, a1 = wl.chunk_range(c)
        s0, s1 = max(a0, t0), min(a1, t1)
        if s0 >= s1:
            continue
        rn = _rng(wl.seed, head, TENSOR[tensor], ROLE["noise"], c)
        noise = rn.standard_normal((a1 - a0, wl.head_dim))[s0 - a0:s1 - a0]
        ro = _rng(wl.seed, head, TENSOR[tensor], ROLE["outlier"], c)
        mag = ro.uniform(lo, hi, (a1 - a0, N_OUTLIER_CH))[s0 - a0:s1 - a0]
        sl = slice(s0 - t0, s1 - t0)
        y[sl] += 0.1 * noise
        reg = region[sl]
        idx = np.arange(s0 - t0, s1 - t0)[:, None]
        y[idx, ch[reg]] += sign[reg] * mag
    return y


def kv_tokens(wl: Workload, tensor: str, t0: int, t1: int, heads=None) -> np.ndarray:
    """float32 [t1 - t0, H, d] K or V values (bf16-exact for bf16 workloads)."""
    heads = range(wl.n_heads) if heads is None else heads
    gen = _tiny_tensor if wl.cid == 1 else _field_tensor
    out = np.stack([gen(wl, h, tensor, t0, t1) for h in heads], axis=1)
    return round_to(out, wl.dtype)


def kv_chunk(wl: Workload, tensor: str, c: int, heads=None) -> np.ndarray:
    """Chunk c of K or V: float32 [N_c, H, d]."""
    t0, t1 = wl.chunk_range(c)
    return kv_tokens(wl, tensor, t0, t1, heads)


def _orthogonal(wl: Workload, head: int) -> np.ndarray:
    r = _rng(wl.seed, head, TENSOR["Q"], ROLE["basis"])
    g = r.standard_normal((wl.head_dim, wl.head_dim))
    qm, rm = np.linalg.qr(g)
    return qm * np.sign(np.diag(rm))[None, :]


def _structured_queries(wl: Workload, head: int, n: int, role: str) -> np.ndarray:
    b = _orthogonal(wl, head)
    r = _rng(wl.seed, head, TENSOR["Q"], ROLE[role])
    a = r.standard_normal((n, wl.head_dim))
    a[:, :8] *= np.sqrt(20.0)
    return a @ b.T


def queries(wl: Workload, heads=None, n: int | None = None) -> np.ndarray:
    """Attending queries float32 [n, H, d] (fp32 or bf16 values)."""
    heads = range(wl.n_heads) if heads is None else heads
    n = wl.n_query if n is None else n
    cols = []
    for h in heads:
        if wl.cid in (4, 5):
            cols.append(_structured_queries(wl, h, n, "query"))
        else:
            cols.append(_rng(wl.seed, h, TENSOR["Q"], ROLE["query"]).standard_normal((n, wl.head_dim)))
    return round_to(np.stack(cols, 1), wl.dtype)


def chunk_queries(wl: Workload, c: int, heads=None) -> np.ndarray:
    """Queries of chunk c's own tokens float32 [N_c, H, d] (bf16 values) for one
    autoregressive step: the workload's query process with a stream per chunk."""
    heads = range(wl.n_heads) if heads is None else heads
    t0, t1 = wl.chunk_range(c)
    cols = []
    for h in heads:
        if wl.cid in (4, 5):
            b = _orthogonal(wl, h)
            a = _rng(wl.seed, h, TENSOR["Q"], ROLE["query"], c + 1).standard_normal((t1 - t0, wl.head_dim))
            a[:, :8] *= np.sqrt(20.0)
            cols.append(a @ b.T)
        else:
            cols.append(_rng(wl.seed, h, TENSOR["Q"], ROLE["query"], c + 1).standard_normal((t1 - t0, wl.head_dim)))
    return round_to(np.stack(cols, 1), "bf16")


def history_queries(wl: Workload, heads=None) -> np.ndarray:
    """History queries float32 [n_hist, H, d] (bf16 values) for QSAC/PSAC statistics."""
    heads = range(wl.n_heads) if heads is None else heads
    n = wl.n_hist or 4096
    return round_to(np.stack([_structured_queries(wl, h, n, "hist") for h in heads], 1), "bf16")
