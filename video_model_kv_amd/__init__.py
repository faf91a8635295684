"""libqkv for MI355X: KV-chunk quantization (k-means smoothing, per-group INT2/INT4,
progressive residual stages, QSAC/PSAC) and attention over the packed cache;
and the practitioner blog's temporally stable 2-bit codec for comparison.

The compute lives in the HIP library ``libqkv.so`` (C-ABI: include/qkv.h); this
package is its thin ctypes binding (``_binding``), helpers that slice a packed
chunk into typed views (``packed``), and the seeded synthetic inputs
(``synth``).
"""
from ._binding import (  # noqa: F401
    Config, QkvError, qkv_attend, qkv_attend_fresh, qkv_chunk_layout, qkv_dequantize, qkv_kmeans_assign,
    qkv_kmeans_update, qkv_last_error, qkv_psac_fit, qkv_quant_pack, qkv_quantize_chunk, qkv_quantize_chunk_noalloc, qkv_quantize_chunks,
    qkv_quantize_chunks_workspace_bytes, qkv_timing_enable, qkv_timing_read, qkv_version, qkv_workspace_bytes, lib, tensor_desc, QKV_FLAG_RTN,
    TConfig, qkv_temporal_layout, qkv_temporal_state_bytes, qkv_temporal_encode, qkv_temporal_decode,
)
