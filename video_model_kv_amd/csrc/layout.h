// Packed-chunk layout, computed identically on the host (qkv_chunk_layout) and
// on the device (the attention kernel rebuilds each chunk's offsets from its
// token count).  The format itself is documented in include/qkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

constexpr int kHeadDim = 128;      // the only head size the library supports
constexpr int kMaxClusters = 256;
constexpr int kMaxStages = 4;
constexpr int kMaxRank = 8;

struct LayoutParams {
  int32_t H, C, n_stages, bits, group, n_int4, psac_rank;
};

// Offsets (bytes from the chunk base) and geometry of one packed chunk.
struct ChunkDecode {
  int H, C, N, n_stages;
  int bits, group, n_int4, int4_words;
  int words, groups;
  const uint8_t* base;
  uint64_t off_codes, stage_codes;
  uint64_t off_scales, stage_scales;
  uint64_t off_labels, stage_labels;
  uint64_t off_centroids, stage_centroids;
  uint64_t off_perm, off_psac;
  int psac_rank;
  uint64_t bytes;
};

__host__ __device__ inline uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

__host__ __device__ inline ChunkDecode make_decode(const LayoutParams& p, int64_t n, const void* base) {
  ChunkDecode d;
  const int n4 = p.n_int4;
  if (n4 > 0) {
    d.int4_words = (n4 * 4 + 31) / 32;
    d.words = d.int4_words + ((128 - n4) * p.bits + 31) / 32;
    d.groups = (n4 + p.group - 1) / p.group + (128 - n4 + p.group - 1) / p.group;
  } else {
    d.int4_words = 0;
    d.words = 128 * p.bits / 32;
    d.groups = 128 / p.group;
  }
  d.H = p.H;
  d.C = p.C;
  d.N = (int)n;
  d.n_stages = p.n_stages;
  d.bits = p.bits;
  d.group = p.group;
  d.n_int4 = n4;
  d.psac_rank = p.psac_rank;
  d.base = reinterpret_cast<const uint8_t*>(base);
  const uint64_t H = (uint64_t)p.H, N = (uint64_t)n, S = (uint64_t)p.n_stages;
  d.stage_codes = align256(H * N * (uint64_t)d.words * 4);
  d.stage_scales = align256(H * N * (uint64_t)d.groups * 2);
  d.stage_labels = align256(H * N);
  d.stage_centroids = align256(H * (uint64_t)p.C * 128 * 2);
  uint64_t off = 0;
  d.off_codes = off;
  off += S * d.stage_codes;
  d.off_scales = off;
  off += S * d.stage_scales;
  d.off_labels = off;
  off += S * d.stage_labels;
  d.off_centroids = off;
  off += S * d.stage_centroids;
  d.off_perm = off;
  if (n4 > 0) off += align256(H * 128);
  d.off_psac = off;
  if (p.psac_rank > 0) off += align256(H * N * (uint64_t)p.psac_rank * 2);
  d.bytes = off;
  return d;
}

}  // namespace qkv
