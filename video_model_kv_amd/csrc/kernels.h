// Internal launch interface between the host API (qkv_host.cpp) and the HIP
// kernels.  Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace qkv {

// A strided [n_tokens][n_heads][128] tensor (dtype 0 = f32, 1 = bf16; 2 = fp16 already scaled by the
// call's operand range: the dense rows of a decoded cache, read by the attention only).
struct TensorView {
  const void* ptr;
  int dtype;
  int64_t n_tokens, stride_token, stride_head;
};

// Channel decode of one head: for original channel k, where its code lives.
//   word index (within the token's words), bit shift, code bits, group index.
struct ChannelCode {
  uint8_t word, shift, bits, group;
};

// ---- k-means (kmeans.hip) ----
// Centroids c: f32 [H][C][128].  The assign forms its MFMA operand, the split
// hi/lo bf16 of fp32(-2 w c), and the weighted norms sum_k w_k c_k^2 (float64,
// rounded to f32) from c in LDS.
// Every launch covers a batch of independent problems (one per grid slice);
// the problems of a batch share dtype, n_tokens, n_heads and n_clusters.
struct KmItem {
  const void* y;                 // tokens [N][H][128] (strided)
  int64_t stride_token, stride_head;
  const float* w;                // QSAC weights [H][128], or null (all ones)
  float* c;
  uint8_t* labels;               // [H][N]
  int* amb_count;                // close calls of the last assign (statistics), or null
  int32_t* counts;               // member counts [H][C] from the update, or null
  uint16_t* cent_bf16;           // bf16 centroids written by launch_centroid_bf16
  int* grp_off;                  // [H][C + 1] cluster offsets from launch_kmeans_group, or null
  uint16_t* grp_list;            // [H][N] tokens ordered by cluster (same producer)
  float* ynorm;                  // [H][N] the assign's ||y||_w^2 of bf16 tokens, kept from the first
                                 // iteration of a stage for the later ones (KmBatch::iter), or null
  // Incremental updates (bf16 tokens, grouped heads), or all null: the exact
  // float64 cluster sums and member counts of the last update, the head's
  // channel magnitude range (the certificate that every subset sum of its
  // tokens is exact in float64), and the labels of the last two updates.
  double* dsum;                  // [H][C][128]
  int32_t* dcnt;                 // [H][C]
  uint32_t* emag;                // [H][2][128]: max magnitude, 0xFFFF - (min nonzero magnitude - 1)
  uint32_t* cert;                // [H]: the head's class (1 float64 sums, 2 64-bit integer sums, 0 neither)
  uint32_t* hlist;               // [2 + 2H]: counts, then the heads of class 0 and of class 2 (k_cert)
  uint8_t* prev;                 // [2][H][N] labels at the previous updates (alternating)
};
constexpr int kKmMaxBatch = 16;
// inc: 0 plain k-means; 1 the first iteration of an incremental stage (the
// update also records dsum, dcnt, emag and the labels); 2 a later iteration
// (heads in a certificate class take launch_kmeans_update_delta, the others
// the full update).  iter: the iteration index (0-based).
struct KmBatch {
  int n, dtype, H, C;
  int64_t N;
  int inc, iter;
  KmItem it[kKmMaxBatch];
};
// Strided initial centroids; clears amb_count and emag.
hipError_t launch_kmeans_init(const KmBatch& b, hipStream_t s);
// Assign = MFMA screening (labels) + float64 re-decision of the close calls,
// in one kernel; adds the number of close calls to amb_count.
hipError_t launch_kmeans_assign(const KmBatch& b, hipStream_t s);
// Update = exact per-cluster sums over the member lists (or label windows) and
// the means.  Zeroes amb_count.
hipError_t launch_kmeans_update(const KmBatch& b, hipStream_t s);
// Counting sort of each head's tokens by label into grp_off / grp_list (heads of
// at most kGroupMaxTokens tokens); the update then reads its clusters' members from there.
constexpr int kGroupMaxTokens = 8192;
hipError_t launch_kmeans_group(const KmBatch& b, hipStream_t s);
// Incremental update (inc == 2): for every head in a certificate class (from
// its first incremental iteration on), the tokens whose label changed since
// the previous update move between the exact sums of their old and new
// clusters; the touched clusters' centroids are rewritten.
hipError_t launch_kmeans_update_delta(const KmBatch& b, hipStream_t s);
// After the first update of an incremental stage: cert[h] from emag.
hipError_t launch_kmeans_cert(const KmBatch& b, hipStream_t s);
// QSAC's residual-range factor (gram.hip): for every problem of the batch,
// w_out[h][k] = fl32(wq[h][k] * fl32(rho * rho)), rho = fl32(max - min) of
// channel k of head h over the problem's tokens.  part: [H][kRangeSplits][2][128]
// f32 per problem (per-split minima and maxima).
constexpr int kRangeSplits = 16;
struct RangeBatch {
  int n, dtype, H;
  int64_t N;
  const void* y[kKmMaxBatch];
  int64_t stride_token[kKmMaxBatch], stride_head[kKmMaxBatch];
  const float* wq[kKmMaxBatch];
  float* w_out[kKmMaxBatch];
  float* part[kKmMaxBatch];
};
hipError_t launch_qsac_range(const RangeBatch& b, hipStream_t s);

// ---- temporally stable 2-bit codec (temporal.hip) ----
// One call codes n_frames consecutive frames (global index frame0 + f) of P
// positions x H heads; frame f's data starts at packed + frame_off[f]: fp16
// values [P][H][128] for an anchor frame, else the sections at the sec_*
// offsets (codes u32 [P][H][4 * bits], lo / scale / oval fp16 [P][H][4], oidx
// u8 [P][H][4]).  State: fb f32 [P][H][128] and anchor fp16 [P][H][128].
constexpr int kTMaxFrames = 64;
struct TCodecArgs {
  int H, P, bits, anchor_every, n_frames;
  float decay;
  int64_t frame0;
  TensorView x;                  // encode input [n_frames * P][H][128]
  float* fb;                     // encode: feedback state (read, then written)
  uint16_t* anchor;              // encode: anchor state; decode: the anchor of frame0's group
  uint8_t* packed;
  uint64_t frame_off[kTMaxFrames];
  int8_t anc_frame[kTMaxFrames];  // decode: the run's frame holding frame f's anchor, -1 = the caller's anchor
  uint64_t sec_codes, sec_lo, sec_scale, sec_oval, sec_oidx;
};
hipError_t launch_temporal_encode(const TCodecArgs& a, hipStream_t s);
hipError_t launch_temporal_decode(const TCodecArgs& a, void* out, int out_dtype, int64_t out_st, int64_t out_sh,
                                  hipStream_t s);
hipError_t launch_centroid_bf16(const KmBatch& b, hipStream_t s);
hipError_t launch_fill_zero_u32(void* p, size_t n_words, hipStream_t s);

// ---- library-held scratch (scratch.hip) ----
// Bytes of the per-device scratch array behind qkv_quantize_chunk_noalloc.
constexpr uint64_t kScratchBytes = 32ull << 20;
// Device address of this device's scratch array (looked up once per device).
hipError_t scratch_of_current_device(void** out);

// ---- quantize / dequantize (quant.hip) ----
struct PackArgs {
  TensorView y;          // stage input
  int H, C, N;
  const uint8_t* labels;       // [H][N]
  const uint16_t* centroids;   // bf16 [H][C][128]
  const uint8_t* perm;         // [H][128] or null (identity)
  int bits, group, n_int4, int4_words;
  uint32_t* codes;             // [H][N][words]
  uint16_t* scales;            // bf16 [H][N][groups]
  int words, groups;
  float* y_next;               // f32 [H][N][128] or null
  uint8_t* perm_out;           // [H][128]: a copy of perm (the chunk's channel order section), or null
};
hipError_t launch_quant_pack(const PackArgs& a, hipStream_t s);
// Several problems of the fast layout (no channel permutation) that share group,
// bits, dtype, H and N, in one launch (grid slice per problem).
struct PackBatch {
  int n;
  PackArgs a[kKmMaxBatch];
};
bool quant_pack_batchable(const PackArgs& a, const PackArgs& b0);
hipError_t launch_quant_pack_batch(const PackBatch& b, hipStream_t s);
// Several problems of the mixed layout (channel permutation, no fp32 residual
// output) that share their geometry, in one launch.
bool quant_pack_mixed_batchable(const PackArgs& a, const PackArgs& b0);
hipError_t launch_quant_pack_mixed_batch(const PackBatch& b, hipStream_t s);

hipError_t launch_dequantize(const ChunkDecode& d, void* out, int out_dtype, int64_t stride_token,
                             int64_t stride_head, hipStream_t s);
hipError_t launch_psac_encode(const ChunkDecode& d, const TensorView& x, const float* U,
                              uint16_t* coef_out, hipStream_t s);
hipError_t launch_copy_perm(const uint8_t* perm, uint8_t* dst, int H, hipStream_t s);

// ---- history-query statistics (gram.hip) ----
hipError_t launch_gram(const TensorView& q, int H, double* partial, int n_split, double* m,
                       hipStream_t s);
// Eigendecomposition of m [H][128][128] (eigh.hip): the rank (at most 8)
// leading eigenvectors into U [H][128][rank], their energy fraction into
// energy [H], m's diagonal into diag [H][128]; rot (rot_bytes, 16-byte
// aligned) is scratch for the rotation record, whose room per head bounds the
// sweeps (invalid value below one sweep's 130,048 bytes per head).
hipError_t launch_eigh(const double* m, int H, void* rot, size_t rot_bytes, int rank, float* U, float* energy,
                       double* diag, hipStream_t s);
// Its diagonal only: m [H][128], the same values as launch_gram's diagonal.
hipError_t launch_gram_diag(const TensorView& q, int H, double* partial, int n_split, double* m,
                            hipStream_t s);

// ---- attention (attend.hip) ----
constexpr int kMaxChunks = 1024;
constexpr int kChunkBatch = 32;      // chunk records per upload launch (fits the kernel-argument limit)
constexpr int kAttendQueries = 256;  // queries per attention workgroup (8 waves of 32)

// Per-chunk record of the concatenated cache (device array in the workspace).
// The section pointers are those of stage 0, head 0; head h adds h * N times
// the per-token size (h * C rows for the centroids).
struct ChunkRec {
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint8_t* kcodes;
  const uint8_t* kscales;
  const uint8_t* klabels;
  const uint8_t* kcent;
  const uint8_t* kpsac;
  const uint8_t* vcodes;
  const uint8_t* vscales;
  const uint8_t* vlabels;
  const uint8_t* vcent;
  const uint8_t* krep;   // mix4 codes of the chunk's keys (64 bytes per token-head, workspace), or null
  int64_t token_start;   // global index of the chunk's first token
  int32_t n;             // tokens in the chunk
  int32_t tile_start;    // global index of the chunk's first 64-key tile
};

// Per 64-key tile of the concatenated cache: the stage-0 section pointers of
// head 0 advanced to the tile's first token (head h adds h * n tokens; the
// centroid pointers are the chunk's tables), and the tile geometry.
struct TileRec {
  const uint8_t* src[2][3];   // [K, V][code words, scales, labels]
  const uint8_t* cent[2];     // [K, V] centroid tables of the chunk
  const uint8_t* kpsac;
  int32_t n;        // tokens in the chunk (head stride in tokens)
  int32_t nvalid;   // keys in the tile (<= 64)
  int32_t kstart;   // global index of the tile's first key
  int32_t token0;   // index of the tile's first key within the chunk
  int32_t chunk;
  int32_t pad;
};
static_assert(sizeof(TileRec) == 96, "TileRec layout");

// Bytes per token of each section (stage 0), for the tile records.
struct TokenBytes {
  int32_t kcodes, vcodes, kscales, vscales, kpsac;
};

// Item order of mixed INT4/INT2 keys on the attention fast path ("mix4"):
// 16 items of 8 positions, each item within one scale group except for at
// most one split on a pair boundary.  rho[r] is the storage position of item
// position r; item i covers groups glo[i] (pairs < jb[i]) and ghi[i] (the
// rest; jb = 4 when glo == ghi).
constexpr int kMix4MaxGroups = 5;
struct MixOrder {
  uint8_t rho[128];
  uint8_t glo[16], ghi[16], jb[16];
};
// The mix4 order of a mixed layout, or false when its groups cannot be laid
// out so (odd class sizes, more than two groups in an item, more than
// kMix4MaxGroups groups per token).
bool mix4_order(const LayoutParams& p, MixOrder* m);

struct ChunkBatch {
  int32_t first, count;
  ChunkRec rec[kChunkBatch];
};
// Uploads one batch of chunk records; the first batch (first == 0) also clears
// the range record.
hipError_t launch_upload_chunks(const ChunkBatch& b, ChunkRec* dst, uint32_t* range, const MixOrder& mix,
                                MixOrder* mix_dst, hipStream_t s);
// mix4 codes of every chunk's keys (ChunkRec::krep) from their packed codes.
hipError_t launch_repack_mix(const ChunkRec* recs, int n_chunks, int max_tokens, const LayoutParams& kp,
                             const MixOrder* mix, hipStream_t s);

// Range record of one attention call (device, kRangeWords words): the largest
// magnitudes of the operands that enter the fp16 MFMAs, as float32 bit patterns
// (non-negative floats order like their bits, so they combine by integer max).
enum RangeSlot { kRgKScale = 0, kRgKCent, kRgVScale, kRgVCent, kRgQ, kRgCoef, kRgQU, kRgKFresh, kRgVFresh, kRangeWords };
// Fills every slot but kRgQU (k_qu adds that one) from the chunks' stored scales,
// centroids and PSAC coefficients, from the queries and from the fresh keys and
// values (n_fresh tokens; none when n_fresh == 0).
hipError_t launch_range_scan(const ChunkRec* recs, int n_chunks, const LayoutParams& kp, const LayoutParams& vp,
                             const TensorView& q, int Nq, const TensorView& kf, const TensorView& vf, int n_fresh,
                             uint32_t* range, hipStream_t s);
// fp16 copies of the chunks' bf16 centroid tables ([chunk][H][C][128]), scaled
// by the tensor's range exponent (2^-e, exact) and rounded to nearest even, for
// the tensors decoded by the attention fast path; k16 / v16 may be NULL (tensor
// not on the fast path).
// Generic-layout caches decoded once into dense fp16 rows dk/dv [Nk][H][128]
// (already scaled by the call's operand range; attended as fresh-chunk tiles
// of dtype 2).
hipError_t launch_dense_decode(const ChunkRec* recs, int n_chunks, int max_n, int H, const LayoutParams& kp,
                               const LayoutParams& vp, const uint32_t* range, uint16_t* dk, uint16_t* dv,
                               hipStream_t s);
hipError_t launch_centroids_f16(const ChunkRec* recs, int n_chunks, const LayoutParams& kp, const LayoutParams& vp,
                                const uint32_t* range, const MixOrder* kmix, uint16_t* k16, uint16_t* v16,
                                hipStream_t s);
// Tile records; the fast-path centroid pointers go to k16 / v16 when given.
// Tiles n_cache_tiles .. n_tiles - 1 are the fresh chunk's (n_fresh tokens,
// the first at global key index fresh_start): chunk = n_chunks, no packed data.
hipError_t launch_tile_table(const ChunkRec* recs, int n_chunks, int n_tiles, int n_cache_tiles, int n_fresh,
                             int64_t fresh_start, TokenBytes tb, int H, int kC, int vC, const uint16_t* k16,
                             const uint16_t* v16, TileRec* tiles, hipStream_t s);

struct AttendArgs {
  TensorView q;
  int H, Nq;
  int64_t Nk;
  int n_chunks, n_tiles;
  LayoutParams kp, vp;           // layouts of the K and V chunks
  const ChunkRec* chunks;        // device [n_chunks]
  const TileRec* tiles;          // device [n_tiles]
  const float* U;                // [H][128][r] or null
  int psac_rank;
  float* qu;                     // workspace [H][Nq][8] f32
  int causal;                    // 1: key j visible to query i iff j < mask_base + (i / mask_F + 1) * mask_F
  int mask_F, mask_base;         // (token-causal: 1 and 0; frame-block over a fresh chunk: frame tokens, cached keys)
  TensorView kf, vf;             // the fresh chunk's keys and values ([Nf][H][128]; ptr null when none)
  int n_cache_tiles;             // tiles of the packed chunks; tiles past them are the fresh chunk's
  float scale;
  int n_split;                   // split s covers tiles [t0 + n*s/n_split, t0 + n*(s+1)/n_split), n = n_tiles - t0
  int tile_lo;                   // t0: the first tile of this launch (0 unless a call takes two launches)
  int split_base, n_split_total; // split s writes partial row split_base + s of n_split_total (1: the output)
  float* part_o;                 // [n_split_total][H][Nq][128]
  float* part_ml;                // [n_split_total][H][Nq][2]
  float* out;                    // [Nq][H][128] via strides
  int64_t out_stride_token, out_stride_head;
  float* logits;                 // [H][Nq][Nk] or null
  uint32_t* range;               // range record (kRangeWords words, see RangeSlot)
  const MixOrder* mixp;          // device copy of the mix4 order (k_mode 2)
  int k_mode;                    // key decode: 0 generic, 1 one uniform INT2 stage (groups of a
                                 // multiple of 32 channels), 2 one mixed INT4/INT2 stage via mix4
  bool v_uniform_int2_1stage;    // value decode: one uniform INT2 stage, groups of a multiple of 32
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace qkv
