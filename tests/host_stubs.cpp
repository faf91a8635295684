// Stand-ins for the kernel launchers and the scratch lookup, for a host-only
// build of libqkv's C-ABI layer (validation, layouts, workspace plans) under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
// Every stand-in reports hipErrorNotSupported: a call that passes validation
// and reaches a launch returns QKV_EDEVICE, which the validation tests never
// expect.
#include "kernels.h"

namespace qkv {

#define QKV_STUB(sig) \
  sig { return hipErrorNotSupported; }

QKV_STUB(hipError_t launch_kmeans_init(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_kmeans_assign(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_kmeans_update(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_kmeans_group(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_kmeans_update_delta(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_kmeans_cert(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_qsac_range(const RangeBatch&, hipStream_t))
QKV_STUB(hipError_t launch_temporal_encode(const TCodecArgs&, hipStream_t))
QKV_STUB(hipError_t launch_temporal_decode(const TCodecArgs&, void*, int, int64_t, int64_t, hipStream_t))
QKV_STUB(hipError_t launch_centroid_bf16(const KmBatch&, hipStream_t))
QKV_STUB(hipError_t launch_fill_zero_u32(void*, size_t, hipStream_t))
QKV_STUB(hipError_t launch_quant_pack(const PackArgs&, hipStream_t))
QKV_STUB(hipError_t launch_quant_pack_batch(const PackBatch&, hipStream_t))
QKV_STUB(hipError_t launch_quant_pack_mixed_batch(const PackBatch&, hipStream_t))
QKV_STUB(hipError_t launch_dequantize(const ChunkDecode&, void*, int, int64_t, int64_t, hipStream_t))
QKV_STUB(hipError_t launch_psac_encode(const ChunkDecode&, const TensorView&, const float*, uint16_t*, hipStream_t))
QKV_STUB(hipError_t launch_copy_perm(const uint8_t*, uint8_t*, int, hipStream_t))
QKV_STUB(hipError_t launch_gram(const TensorView&, int, double*, int, double*, hipStream_t))
QKV_STUB(hipError_t launch_gram_diag(const TensorView&, int, double*, int, double*, hipStream_t))
QKV_STUB(hipError_t launch_eigh(const double*, int, void*, size_t, int, float*, float*, double*, hipStream_t))
QKV_STUB(hipError_t launch_dense_decode(const ChunkRec*, int, int, int, const LayoutParams&, const LayoutParams&,
                                        const uint32_t*, uint16_t*, uint16_t*, hipStream_t))
QKV_STUB(hipError_t launch_upload_chunks(const ChunkBatch&, ChunkRec*, uint32_t*, const MixOrder&, MixOrder*, hipStream_t))
QKV_STUB(hipError_t launch_repack_mix(const ChunkRec*, int, int, const LayoutParams&, const MixOrder*, hipStream_t))
QKV_STUB(hipError_t launch_range_scan(const ChunkRec*, int, const LayoutParams&, const LayoutParams&, const TensorView&,
                                      int, const TensorView&, const TensorView&, int, uint32_t*, hipStream_t))
QKV_STUB(hipError_t launch_centroids_f16(const ChunkRec*, int, const LayoutParams&, const LayoutParams&, const uint32_t*,
                                         const MixOrder*, uint16_t*, uint16_t*, hipStream_t))
QKV_STUB(hipError_t launch_tile_table(const ChunkRec*, int, int, int, int, int64_t, TokenBytes, int, int, int,
                                      const uint16_t*, const uint16_t*, TileRec*, hipStream_t))
QKV_STUB(hipError_t launch_attend(const AttendArgs&, hipStream_t))
QKV_STUB(hipError_t scratch_of_current_device(void**))

bool quant_pack_batchable(const PackArgs&, const PackArgs&) { return false; }
bool quant_pack_mixed_batchable(const PackArgs&, const PackArgs&) { return false; }

}  // namespace qkv
