"""Typed views into a packed chunk (a uint8 device tensor), by the offsets that
qkv_chunk_layout reports.  Pure slicing: no arithmetic of the method."""
from __future__ import annotations

from ._binding import Config, qkv_chunk_layout


def views(packed, cfg: Config, n_tokens: int) -> dict:
    """{'codes': [L][H][N][W] int32, 'scales': [L][H][N][G] int16 (bf16 bits),
    'labels': [L][H][N] uint8, 'centroids': [L][H][C][128] int16 (bf16 bits),
    'perm': [H][128] uint8 or None, 'psac': [H][N][r] int16 (bf16 bits) or None}."""
    import torch
    L = qkv_chunk_layout(cfg, n_tokens)
    H, N, C, S = cfg.n_heads, n_tokens, cfg.n_clusters, cfg.n_stages
    W, G = L.words_per_token, L.groups_per_token

    def sl(off, nbytes):
        return packed[off:off + nbytes]

    out = {"layout": L}
    out["codes"] = torch.stack([sl(L.off_codes + l * L.stage_bytes_codes, H * N * W * 4).view(torch.int32)
                                .view(H, N, W) for l in range(S)])
    out["scales"] = torch.stack([sl(L.off_scales + l * L.stage_bytes_scales, H * N * G * 2).view(torch.int16)
                                 .view(H, N, G) for l in range(S)])
    out["labels"] = torch.stack([sl(L.off_labels + l * L.stage_bytes_labels, H * N).view(H, N) for l in range(S)])
    out["centroids"] = torch.stack([sl(L.off_centroids + l * L.stage_bytes_centroids, H * C * 128 * 2)
                                    .view(torch.int16).view(H, C, 128) for l in range(S)])
    out["perm"] = sl(L.off_perm, H * 128).view(H, 128) if cfg.n_int4_channels > 0 else None
    r = cfg.psac_rank
    out["psac"] = sl(L.off_psac, H * N * r * 2).view(torch.int16).view(H, N, r) if r > 0 else None
    return out
