// Attention computed directly over the packed KV cache.
//
// Method: Quant VideoGen notes, "Key designs / Algorithm-system co-design"
// (quantization/dequantization fused with the attention kernel, 2-bit codes
// packed as integers) and "Method / Overall framework" (x_hat = S q + C_i);
// QuantWM summary, "QuantWM", second technique (PSAC: the stored projections of
// the key error on the query principal subspace U are added back to the logits,
// s += (q U) . coef).
//
// Work decomposition: one workgroup (8 waves, 512 threads) per (head, key
// split, 256-query tile).  A key split is a contiguous run of 64-key tiles of
// the concatenated chunks (a tile never straddles two chunks).  Per key tile the
// workgroup decodes K_hat and V_hat^T into LDS once for its 256 queries, then
// each wave (32 queries) computes S^T = K_hat Q^T and O^T += V_hat^T P^T on
// MFMA (v_mfma_f32_32x32x16_f16) with an online softmax in the exp2 domain.
//
// Numerics: K_hat and V_hat enter the MFMAs as fp16 (S q + C evaluated by one
// packed fp16 FMA on the fast paths; in fp32 and rounded once on the generic
// ones).  A range pre-pass finds the largest stored scale, centroid, PSAC
// coefficient and query of the call, and each operand class is scaled by a
// power of two 2^-e (e >= 0, exact) that keeps every fp16 operand and decoded
// value finite; the logits and outputs are scaled back (e = 0, no change, for
// caches within the fp16 range).  bf16 queries convert to fp16 exactly between
// 2^-14 and 65504 in magnitude (rounded below); fp32 queries are split into fp16 hi + lo (two MFMA passes).
// Probabilities are rounded to fp16 for P V (fp32 accumulation) and the row
// sums use the same rounded values.  The PSAC term rides one extra MFMA
// k-step: [coef | coef] against [hi(qU) | lo(qU)].  Splits are merged with the
// usual log-sum-exp rescaling.
#include <algorithm>
#include <climits>
#include <cstddef>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

constexpr int kKTile = 64;      // keys per tile
constexpr int kKPitch = 136;    // bf16 pitch of the K_hat rows in LDS
constexpr int kVPitch = 66;     // fp16 pitch of the V_hat^T rows in LDS (33 dwords: odd, for conflict-free writes)
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kHeadDim == 128, "scale indexes below divide by the head size with a shift by 7");

__device__ __forceinline__ const uint8_t* sp(const ChunkDecode& d, uint64_t off, uint64_t stride, int l) {
  return d.base + off + stride * (uint64_t)l;
}

__device__ __forceinline__ ChannelCode code_at(int p, int bits, int group, int n_int4, int int4_words) {
  ChannelCode cc;
  int pos, b, w0, gidx;
  if (n_int4 > 0 && p < n_int4) {
    pos = p; b = 4; w0 = 0; gidx = p / group;
  } else if (n_int4 > 0) {
    pos = p - n_int4; b = bits; w0 = int4_words;
    gidx = (n_int4 + group - 1) / group + pos / group;
  } else {
    pos = p; b = bits; w0 = 0; gidx = p / group;
  }
  const int per = 32 / b;
  cc.word = (uint8_t)(w0 + pos / per);
  cc.shift = (uint8_t)(b * (pos % per));
  cc.bits = (uint8_t)b;
  cc.group = (uint8_t)gidx;
  return cc;
}

// Decode table of head h (block-cooperative; the caller synchronises).  A perm
// that is not a permutation decodes wrongly but stays inside every buffer.
__device__ __forceinline__ void build_tab(const ChunkDecode& d, int h, ChannelCode* tab) {
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) tab[p] = ChannelCode{0, 0, (uint8_t)d.bits, 0};
  __syncthreads();
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) {
    const int k = d.n_int4 > 0 ? ((int)(d.base + d.off_perm)[h * kHeadDim + p] & (kHeadDim - 1)) : p;
    tab[k] = code_at(p, d.bits, d.group, d.n_int4, d.int4_words);
  }
}

// Generic decode: x_hat of token j (within the chunk), channels k0..k0+NCH-1.
template <int NCH>
__device__ __forceinline__ void decode_generic(const ChunkDecode& d, const ChannelCode* tab, int h, int j,
                                               int k0, float* v) {
#pragma unroll
  for (int e = 0; e < NCH; ++e) v[e] = 0.0f;
  for (int l = 0; l < d.n_stages; ++l) {
    const int64_t row = (int64_t)h * d.N + j;
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(sp(d, d.off_codes, d.stage_codes, l)) + row * d.words;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(sp(d, d.off_scales, d.stage_scales, l)) + row * d.groups;
    const int lab = min((int)sp(d, d.off_labels, d.stage_labels, l)[row], d.C - 1);
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(sp(d, d.off_centroids, d.stage_centroids, l)) +
                           ((int64_t)h * d.C + lab) * kHeadDim + k0;
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const ChannelCode cc = tab[k0 + e];
      const uint32_t u = (codes[cc.word] >> cc.shift) & ((1u << cc.bits) - 1u);
      const float q = (float)((int)u - (1 << (cc.bits - 1)));
      const float yhat = __fadd_rn(bf16_bits_to_f32(scales[cc.group]) * q, bf16_bits_to_f32(crow[e]));
      v[e] = l == 0 ? yhat : __fadd_rn(v[e], yhat);
    }
  }
}

// Uniform layout (no channel permutation): the same x_hat as decode_generic
// for channels k0 .. k0 + NCH - 1 (k0 a multiple of NCH, so they share one
// code word and one scale group in every stage).  The stage loop runs to
// kMaxStages with clamped stage indexes so that every load is issued before
// any value is used -- the labels of all stages, then the code words, scales
// and centroid pieces they select -- instead of two dependent round trips per
// stage; stages past n_stages are loaded again from the last one and not added.
template <int NCH>
__device__ __forceinline__ void decode_uniform(const ChunkDecode& d, int h, int j, int k0, float* v) {
  static_assert(NCH == 8 || NCH == 4, "channels per item");
  const int64_t row = (int64_t)h * d.N + j;
  const int per = 32 / d.bits;
  int lab[kMaxStages];
#pragma unroll
  for (int l = 0; l < kMaxStages; ++l) lab[l] = sp(d, d.off_labels, d.stage_labels, min(l, d.n_stages - 1))[row];
  uint32_t word[kMaxStages], sc[kMaxStages], cw[kMaxStages][NCH / 2];
#pragma unroll
  for (int l = 0; l < kMaxStages; ++l) {
    const int ls = min(l, d.n_stages - 1);
    word[l] = reinterpret_cast<const uint32_t*>(sp(d, d.off_codes, d.stage_codes, ls))[row * d.words + k0 / per];
    sc[l] = reinterpret_cast<const uint16_t*>(sp(d, d.off_scales, d.stage_scales, ls))[row * d.groups + k0 / d.group];
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(sp(d, d.off_centroids, d.stage_centroids, ls)) +
                           ((int64_t)h * d.C + min(lab[l], d.C - 1)) * kHeadDim + k0;
    if constexpr (NCH == 8) {
      const uint4 c = *reinterpret_cast<const uint4*>(crow);
      cw[l][0] = c.x; cw[l][1] = c.y; cw[l][2] = c.z; cw[l][3] = c.w;
    } else {
      const uint2 c = *reinterpret_cast<const uint2*>(crow);
      cw[l][0] = c.x; cw[l][1] = c.y;
    }
  }
  const int sh0 = d.bits * (k0 % per);
  const uint32_t mask = (1u << d.bits) - 1u;
  const int off = 1 << (d.bits - 1);
#pragma unroll
  for (int l = 0; l < kMaxStages; ++l) {
    if (l < d.n_stages) {
      const float S = bf16_bits_to_f32(sc[l]);
#pragma unroll
      for (int e = 0; e < NCH; ++e) {
        const float q = (float)((int)((word[l] >> (sh0 + d.bits * e)) & mask) - off);
        const float yhat = __fadd_rn(S * q, bf16_bits_to_f32((cw[l][e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
        v[e] = l == 0 ? yhat : __fadd_rn(v[e], yhat);
      }
    }
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;                 // two waves per SIMD
constexpr int kBM = kWaves * 32;          // queries per workgroup, 32 per wave
constexpr int kThreads = kWaves * 64;
constexpr int kItems = 1024 / kThreads;   // K (and V) decode items per thread per tile
constexpr int kRing = 3;                  // raw-tile slots in LDS
constexpr int kMetaSlots = 6;             // tile-record slots in LDS
constexpr float kF16Max = 65504.0f;
static_assert(kBM == kAttendQueries, "queries per workgroup");

// ---- operand range ----
// Every decoded key or value is a sum over stages of S q + C with |q| <= 2^(b-1),
// so n_stages * (2^(b-1) max|S| + max|C|) bounds it.  The exponent of a tensor
// is the smallest e >= 0 that brings its bounds under kRangeLimit, which sits
// below the fp16 maximum by more than the fp16 roundings of S and C can add.
constexpr float kRangeLimit = 65024.0f;

__device__ __forceinline__ int range_exp(float x) {
  if (!(x > kRangeLimit)) return 0;
  if (!(x < 3.0e38f)) return 120;
  int k;
  const float m = frexpf(x / kRangeLimit, &k);      // ratio = m 2^k, m in [0.5, 1)
  return m == 0.5f ? k - 1 : k;
}

struct RangeExps {
  int ek, ev, eq;
};

__device__ __forceinline__ float code_bound(const LayoutParams& p, float smax, float cmax) {
  const float qmax = (p.n_int4 > 0 || p.bits == 4) ? 8.0f : 2.0f;
  return (float)p.n_stages * (qmax * smax + cmax);
}

// rg: the call's range record (see RangeSlot); psac: the key PSAC term is on.
template <typename P>
__device__ __forceinline__ RangeExps range_exps(P rg, const LayoutParams& kp, const LayoutParams& vp, bool psac) {
  RangeExps e;
  e.ek = range_exp(code_bound(kp, __uint_as_float(rg[kRgKScale]), __uint_as_float(rg[kRgKCent])));
  e.ev = range_exp(code_bound(vp, __uint_as_float(rg[kRgVScale]), __uint_as_float(rg[kRgVCent])));
  e.eq = range_exp(__uint_as_float(rg[kRgQ]));
  e.ek = max(e.ek, range_exp(__uint_as_float(rg[kRgKFresh])));   // a fresh chunk's keys and values enter as they are
  e.ev = max(e.ev, range_exp(__uint_as_float(rg[kRgVFresh])));
  if (psac) {
    e.ek = max(e.ek, range_exp(__uint_as_float(rg[kRgCoef])));
    e.eq = max(e.eq, range_exp(__uint_as_float(rg[kRgQU])));
  }
  return e;
}

__device__ __forceinline__ float pow2(int e) { return __builtin_ldexpf(1.0f, e); }

// two fp32 values -> packed fp16 (round to nearest even), saturated to the fp16 range
__device__ __forceinline__ uint32_t pack_f16x2(float x0, float x1) {
  f16x2 r;
  r[0] = (_Float16)__builtin_amdgcn_fmed3f(x0, -kF16Max, kF16Max);
  r[1] = (_Float16)__builtin_amdgcn_fmed3f(x1, -kF16Max, kF16Max);
  return __builtin_bit_cast(uint32_t, r);
}

// Two 2-bit codes (already spread to bits [0,1] and [16,17] of x) -> fp16 pair
// (u0 - 2, u1 - 2): 0x6400 | u is the fp16 number 1024 + u.
__device__ __forceinline__ f16x2 codes_to_f16x2(uint32_t x) {
  const f16x2 biased = __builtin_bit_cast(f16x2, x | 0x64006400u);
  const f16x2 off = {(_Float16)1026.0f, (_Float16)1026.0f};
  return biased - off;
}
// S * q + c as fp16 pairs for NP consecutive channel pairs: code pair j of `t`
// sits at bits [4j, 4j+1] and [4j+16, 4j+17] (t = codes | codes << 14); cw holds
// the centroid pairs already in fp16 (the per-call fp16 copy of the chunk's
// bf16 table).  S and the centroids arrive scaled by the keys' or values' range
// exponent, so |S q + c| stays below the fp16 maximum without a clamp.
template <int NP>
__device__ __forceinline__ void decode_pairs_f16(uint32_t t, float S, const uint32_t* cw, uint32_t* out) {
  const _Float16 sh = (_Float16)S;
  const f16x2 s2 = {sh, sh};
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const f16x2 q = codes_to_f16x2((t >> (4 * j)) & 0x00030003u);
    out[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(s2, q, __builtin_bit_cast(f16x2, cw[j])));
  }
}

// max(x, x of lane ^ 32): v_permlane32_swap exchanges the two 32-lane halves
// of its operands in registers (no LDS round trip); whichever of its two
// results holds the other half's value, the three-way max takes it.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Asynchronous global -> LDS copy: every active lane moves BYTES bytes from its
// own address to dst + lane * BYTES (dst is wave-uniform).  Tracked by vmcnt.
template <int BYTES>
__device__ __forceinline__ void dma(const void* src, void* dst) {
  const glb_ptr g = (glb_ptr)const_cast<void*>(src);
  if constexpr (BYTES == 16) __builtin_amdgcn_global_load_lds(g, (lds_ptr)dst, 16, 0, 0);
  else if constexpr (BYTES == 4) __builtin_amdgcn_global_load_lds(g, (lds_ptr)dst, 4, 0, 0);
  else if constexpr (BYTES == 2) __builtin_amdgcn_global_load_lds(g, (lds_ptr)dst, 2, 0, 0);
  else __builtin_amdgcn_global_load_lds(g, (lds_ptr)dst, 1, 0, 0);
  static_assert(BYTES == 16 || BYTES == 4 || BYTES == 2 || BYTES == 1, "copy size");
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

typedef const __attribute__((address_space(4))) ChunkRec* crec_ptr;
typedef const __attribute__((address_space(4))) TileRec* ctile_ptr;
typedef const __attribute__((address_space(4))) AttendArgs* cargs_ptr;
typedef const __attribute__((address_space(4))) uint32_t* crange_ptr;


// Mixed INT4/INT2 keys on the fast path ("mix4"): a pre-pass (k_repack_mix)
// rewrites each key's codes as 128 nibbles u' = q + 8 in the per-call item
// order of MixOrder (whole 8-position items of one scale group, the groups'
// remainders packed into the last items, each item split at most once, on a
// pair boundary), with the two codes of a pair at nibble slots j and j + 4 of
// the item's word.  Decoded keys then sit in LDS in that order; the queries are
// loaded in the same order (through the chunk's channel permutation), so the
// dot products are unchanged.
__device__ __forceinline__ void decode_mix4(uint32_t w, float slo, float shi, int jb, const uint32_t* cw,
                                            uint32_t* out) {
  const _Float16 lo = (_Float16)slo, hi = (_Float16)shi;
  const f16x2 slo2 = {lo, lo}, shi2 = {hi, hi};
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 q = __builtin_bit_cast(f16x2, ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u) - off;
    const f16x2 s2 = j < jb ? slo2 : shi2;
    out[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(s2, q, __builtin_bit_cast(f16x2, cw[j])));
  }
}

// NCH values of a fresh-chunk row (token tok, head h, channels k0 ..), as float.
template <int NCH>
__device__ __forceinline__ void fresh_row(const TensorView& t, int tok, int h, int k0, float* v) {
  const int64_t off = (int64_t)tok * t.stride_token + (int64_t)h * t.stride_head + k0;
  if (t.dtype == 0) {
    const float* p = reinterpret_cast<const float*>(t.ptr) + off;
#pragma unroll
    for (int e = 0; e < NCH; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + e);
      v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(t.ptr) + off;
    uint32_t w[NCH / 2];
    if constexpr (NCH == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x; w[1] = x.y;
    }
#pragma unroll
    for (int e = 0; e < NCH; ++e) v[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
  }
}

// KM: key decode mode -- 0 generic (every layout), 1 one uniform INT2 stage,
// 2 one mixed INT4/INT2 stage through the mix4 pre-pass.
// FRESH: the keys end with a fresh chunk (unquantized rows, frame-block mask).
template <bool QF32, int KM, bool VFAST, bool LOGITS, bool PSAC, bool FRESH>
__global__ __launch_bounds__(kThreads) void k_attend(AttendArgs a) {
  constexpr bool KFAST = KM != 0;                // keys through the copy ring and the LDS staging
  static_assert(!FRESH || !QF32, "fresh chunks: bf16 queries");
  static_assert(KM != 2 || (!QF32 && !PSAC), "mix4 keys: bf16 queries, no PSAC term");
  constexpr int kKW = KM == 2 ? 16 : 8;          // K code words per key in the ring
  constexpr int kKGm = KM == 2 ? kMix4MaxGroups : 4;   // K scale groups per key (at most)
  // Separate LDS objects: the compiler waits for outstanding asynchronous
  // copies before an LDS read only when the read may touch a copy target, so
  // the MFMA operands (K, Vt, Kp) live apart from the copy targets (ring and
  // centroid staging), and the labels (written by plain stores) apart again.
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKTile][kKPitch];         // fp16 K_hat rows
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][kHeadDim][kVPitch];      // fp16 V_hat^T rows
  __shared__ __attribute__((aligned(16))) uint16_t sKp[2][kKTile][16];             // fp16 [coef | coef]
  __shared__ __attribute__((aligned(16))) uint16_t sCentK[2][kKTile * kHeadDim];   // gathered K centroid rows
  __shared__ __attribute__((aligned(16))) uint16_t sCentV[2][kKTile * kHeadDim];   // gathered V centroid rows
  __shared__ __attribute__((aligned(16))) uint32_t sRcK[kRing][kKTile * kKW];      // [slot] K code words
  __shared__ __attribute__((aligned(16))) uint32_t sRcV[kRing][kKTile * 8];        // [slot] V code words
  __shared__ __attribute__((aligned(16))) uint16_t sRsK[kRing][kKTile * kKGm + 8]; // [slot] K scales (+ lead)
  __shared__ __attribute__((aligned(16))) uint16_t sRsV[kRing][kKTile * 4 + 8];    // [slot] V scales (+ lead)
  __shared__ __attribute__((aligned(8))) uint8_t sRho[KM == 2 ? kHeadDim : 8];    // mix4 item order
  __shared__ __attribute__((aligned(16))) uint8_t sRl[kRing][2][kKTile + 16];      // [slot][K/V] labels (+ lead)
  __shared__ ChannelCode sTabK[kHeadDim], sTabV[kHeadDim];                         // generic decode tables
  __shared__ __attribute__((aligned(16))) uint32_t sMeta[kMetaSlots][sizeof(TileRec) / 4];   // tile records

  const int q_tiles = (a.Nq + kBM - 1) / kBM;
  const uint32_t total = (uint32_t)(q_tiles * a.n_split * a.H);
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int qt = logical % q_tiles;
  const int split = (logical / q_tiles) % a.n_split;
  const int h = logical / (q_tiles * a.n_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                   // the two waves of a SIMD sit in different groups
  const int col = lane & 31, half = lane >> 5;
  const int q_last = min(a.Nq, (qt + 1) * kBM) - 1;
  const int wq_first = qt * kBM + wave * 32;   // this wave's queries
  const int wq_last = min(a.Nq, wq_first + 32) - 1;
  const bool wave_active = wq_first < a.Nq;
  const int qrow = wq_first + col;             // this lane's query
  const bool qok = qrow < a.Nq;
  // visibility (causal modes): key j is visible to query i iff j < vis_end(i)
  // (token-causal: i + 1; with a fresh chunk: mask_base + (i / F + 1) F)
  auto vis_end = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr (FRESH) return a.mask_base + (i / a.mask_F + 1) * a.mask_F;
    return i + 1;
  };

  // operand scaling of this call (scalar loads of the range record)
  const RangeExps rx = range_exps((crange_ptr)a.range, a.kp, a.vp, PSAC);
  const float qsc = pow2(-rx.eq), ksc = pow2(-rx.ek), vsc = pow2(-rx.ev);
  uint32_t mdesc = 0;                            // mix4: this thread's item (first group, last group, split pair)
  if constexpr (KM == 2) {
    const int it = tid & 15;
    mdesc = (uint32_t)a.mixp->glo[it] | ((uint32_t)a.mixp->ghi[it] << 8) | ((uint32_t)a.mixp->jb[it] << 16);
  }

  // ---- Q fragments in fp16 (B operand: column = query, k = channel) ----
  f16x8 qh[8];
  f16x8 ql[QF32 ? 8 : 1];
  f16x8 qpsac;
  if constexpr (KM == 2) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qh[s] = f16x8{};   // loaded in item order with the first tile's chunk
  } else {
    const int64_t base = (int64_t)(qok ? qrow : 0) * a.q.stride_token + (int64_t)h * a.q.stride_head;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = s * 16 + half * 8;
      float v[8];
      if constexpr (QF32) {
        const float* p = reinterpret_cast<const float*>(a.q.ptr) + base + ch;
        float4 x0 = *reinterpret_cast<const float4*>(p);   // p is in range (query 0 when !qok)
        float4 x1 = *reinterpret_cast<const float4*>(p + 4);
        if (!qok) x0 = x1 = make_float4(0, 0, 0, 0);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w; v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(a.q.ptr) + base + ch;
        uint4 r = *reinterpret_cast<const uint4*>(p);      // p is in range (query 0 when !qok)
        if (!qok) r = make_uint4(0, 0, 0, 0);
        const uint32_t r4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((r4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
      f16x8 hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = __builtin_amdgcn_fmed3f(v[e] * qsc, -kF16Max, kF16Max);
        hi[e] = (_Float16)v[e];
      }
      qh[s] = hi;
      if constexpr (QF32) {
        f16x8 lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = (_Float16)(v[e] - (float)hi[e]);
        ql[QF32 ? s : 0] = lo;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.0f;
      if (PSAC && qok && e < a.psac_rank)
        v = __builtin_amdgcn_fmed3f(a.qu[((int64_t)h * a.Nq + qrow) * kMaxRank + e] * qsc, -kF16Max, kF16Max);
      const _Float16 hv = (_Float16)v;
      qpsac[e] = half == 0 ? hv : (_Float16)(v - (float)hv);
    }
  }
  if constexpr (KM == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qpsac[e] = (_Float16)0.0f;
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;       // m_run: running max in the scaled (log2) domain
  const float sfull = a.scale * pow2(rx.eq + rx.ek);   // logit = sfull * accumulator
  const float c2 = sfull * kLog2e;

  const int64_t t_span = a.n_tiles - a.tile_lo;
  const int t_begin = a.tile_lo + (int)((t_span * split) / a.n_split);
  int t_end = a.tile_lo + (int)((t_span * (split + 1)) / a.n_split);
  const int prow_split = a.split_base + split;   // this split's partial row

  // Tile and chunk records are read-only here: scalar loads through the
  // constant address space keep them out of the vector-memory counter, which
  // the asynchronous copies below are waited on with.
  const crec_ptr recs = (crec_ptr)a.chunks;
  const ctile_ptr tiles = (ctile_ptr)a.tiles;

  // causal: drop trailing tiles wholly above the diagonal (unless debug logits are requested)
  if (a.causal && !LOGITS) {
    while (t_end > t_begin && tiles[t_end - 1].kstart >= vis_end(q_last)) --t_end;
  }
  if (t_begin >= t_end) {
    // nothing visible in this split: write an empty partial
    if (qok && a.n_split_total > 1) {
      if (half == 0) {
        float* ml = a.part_ml + (((int64_t)prow_split * a.H + h) * a.Nq + qrow) * 2;
        ml[0] = -INFINITY;
        ml[1] = 0.0f;
      }
      float* prow = a.part_o + (((int64_t)prow_split * a.H + h) * a.Nq + qrow) * kHeadDim;
      for (int d0 = half * 4; d0 < kHeadDim; d0 += 8)
        *reinterpret_cast<float4*>(prow + d0) = make_float4(0, 0, 0, 0);
    }
    return;
  }

  // ---- tile pipeline ----
  // Four stages, one tile each, one barrier per step:
  //   (1) raw copy: code words, scales and labels -> LDS ring (asynchronous);
  //   (2) centroid gather: the labelled centroid rows -> LDS staging (asynchronous);
  //   (3) decode: K_hat rows and V_hat^T rows in fp16 -> LDS buffer;
  //   (4) compute: S^T = K_hat Q^T, online softmax, O^T += V_hat^T P^T.
  // At step i the workgroup runs (1) on tile i+3, (2) on i+2, (3) on i+1 and (4)
  // on i.  Waves 0-3 compute before they decode, waves 4-7 decode before they
  // compute, so the two waves sharing a SIMD overlap MFMA and VALU work.
  //
  // Per-thread and per-wave indexes used inside the steps come from xtid and
  // xwave, which are made opaque at every step (xtid only in the variants
  // whose registers cannot hold the lane addresses) so that the addresses
  // derived from them are recomputed there instead of being held in registers
  // across the whole loop.
  int xtid = tid, xwave = wave;
  auto geom = [&](int cc, bool v) __attribute__((always_inline)) -> ChunkDecode {
    return make_decode(v ? a.vp : a.kp, recs[cc].n, v ? recs[cc].vbase : recs[cc].kbase);
  };
  const int kG = kHeadDim / a.kp.group, vG = kHeadDim / a.vp.group;   // scale groups per token (fast paths)
  const int kGs = __builtin_ctz(kG), vGs = __builtin_ctz(vG);
  const int kGn = KM == 2 ? make_decode(a.kp, 1, nullptr).groups : kG;  // K scales per key in the ring
  constexpr int kKBpk = KM == 2 ? 64 : 32;       // K code bytes per key in the ring
  const int kC = a.kp.C, vC = a.vp.C;

  // Tile records travel into an LDS ring (sMeta, kMetaSlots tiles) by
  // asynchronous copy five tiles ahead of their first use, so that a step
  // reads them from LDS instead of taking scalar-cache misses.  A step reads
  // the fields it needs at its start into small views; the view of a tile past
  // the end of the split has nvalid = 0.  Scale and label runs of a head need
  // not start on a 4-byte boundary: they are copied from the boundary below
  // and sit `lead` bytes into their LDS slot.
  constexpr int kRecWords = (int)(sizeof(TileRec) / 4);
  constexpr int kFSrc = 0, kFCent = 12, kFPsac = 16, kFN = 18, kFNvalid = 19, kFKstart = 20, kFChunk = 22;
  static_assert(offsetof(TileRec, cent) == 4 * kFCent && offsetof(TileRec, kpsac) == 4 * kFPsac &&
                offsetof(TileRec, n) == 4 * kFN && offsetof(TileRec, nvalid) == 4 * kFNvalid &&
                offsetof(TileRec, kstart) == 4 * kFKstart && offsetof(TileRec, chunk) == 4 * kFChunk,
                "TileRec field offsets");
  auto meta_copy = [&](int j) __attribute__((always_inline)) {   // wave 0 only
    const int lane = xtid & 63;
    if (lane < kRecWords)
      dma<4>(reinterpret_cast<const uint8_t*>(a.tiles + j) + lane * 4, &sMeta[j % kMetaSlots][0]);
  };
  auto m32 = [&](int j, int k) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)sMeta[j % kMetaSlots][k]);
  };
  auto m64 = [&](int j, int k) __attribute__((always_inline)) -> const uint8_t* {
    return reinterpret_cast<const uint8_t*>(((uint64_t)m32(j, k + 1) << 32) | m32(j, k));
  };
  auto lead_of = [](uint32_t addr_lo) __attribute__((always_inline)) -> int { return (int)(addr_lo & 3); };
  // raw copy role of this wave: tensor rv, part rpart (code words by parts
  // 0 and 1, scales by part 2, labels by part 3); bpk = bytes per key
  struct RawRole {
    int rv, rpart, rsel, bpk;
  };
  auto raw_role = [&]() __attribute__((always_inline)) -> RawRole {
    RawRole q;
    q.rv = xwave >> 2;
    q.rpart = xwave & 3;
    q.rsel = q.rpart < 2 ? 0 : q.rpart - 1;
    q.bpk = q.rsel == 0 ? (q.rv ? 32 : kKBpk) : q.rsel == 1 ? 2 * (q.rv ? vG : kGn) : 1;
    return q;
  };
  struct RawView {                               // tile i+3: this wave's run
    const uint8_t* src;
    int nvalid;
  };
  struct GatherView {                            // tile i+2
    const uint8_t* cent[2];
    int lead[2], nvalid;
  };
  struct DecodeView {                            // tile i+1
    int lead[2], nvalid;                         // lead in scales (2 bytes)
    int fresh, ftok0;                            // a fresh-chunk tile and its first token there
  };
  auto raw_view = [&](int j, bool live) __attribute__((always_inline)) -> RawView {
    const RawRole q = raw_role();
    RawView w;
    const int64_t hrow = (int64_t)h * (int)m32(j, kFN);
    w.src = m64(j, kFSrc + (q.rv * 3 + q.rsel) * 2) + hrow * q.bpk + (q.rpart == 1 ? 32 * q.bpk : 0);
    w.nvalid = live ? (int)m32(j, kFNvalid) : 0;
    return w;
  };
  auto gather_view = [&](int j, bool live) __attribute__((always_inline)) -> GatherView {
    GatherView w;
    const uint32_t hrow = (uint32_t)h * m32(j, kFN);
    w.cent[0] = m64(j, kFCent) + (int64_t)h * kC * kHeadDim * 2;
    w.cent[1] = m64(j, kFCent + 2) + (int64_t)h * vC * kHeadDim * 2;
    w.lead[0] = lead_of(m32(j, kFSrc + 4) + hrow);         // src[0][2]: K labels
    w.lead[1] = lead_of(m32(j, kFSrc + 10) + hrow);        // src[1][2]: V labels
    w.nvalid = live ? (int)m32(j, kFNvalid) : 0;
    return w;
  };
  auto decode_view = [&](int j, bool live) __attribute__((always_inline)) -> DecodeView {
    DecodeView w;
    const uint32_t hrow = (uint32_t)h * m32(j, kFN);
    w.lead[0] = lead_of(m32(j, kFSrc + 2) + hrow * (uint32_t)(2 * kGn)) >> 1;   // src[0][1]: K scales
    w.lead[1] = lead_of(m32(j, kFSrc + 8) + (hrow << (vGs + 1))) >> 1;   // src[1][1]: V scales
    w.nvalid = live ? (int)m32(j, kFNvalid) : 0;
    w.fresh = FRESH && j >= a.n_cache_tiles;
    w.ftok0 = FRESH ? (j - a.n_cache_tiles) * kKTile : 0;
    return w;
  };

  // (1) raw copy into ring slot r: waves 0-3 copy K, waves 4-7 V (code words
  // by two waves, scales and labels by one each), all by asynchronous 16- or
  // 4-byte copies.
  auto raw_copy = [&](const RawView& R, int r) __attribute__((always_inline)) {
    const int lane = xtid & 63;
    const RawRole q = raw_role();
    const int rv = q.rv, rpart = q.rpart, rsel = q.rsel, bpk = q.bpk;
    if ((rv == 0 && !KFAST) || (rv == 1 && !VFAST)) return;
    if (rsel == 0) {                             // code words of 32 keys: 32 (or 64 for mix4 keys) bytes each
      uint32_t* dst = rv ? &sRcV[r][rpart * 256] : &sRcK[r][rpart * 32 * kKW];   // 32 keys per part
#pragma unroll
      for (int x = 0; x < kKBpk / 32; ++x) {
        if (x * 32 < bpk) {                      // wave-uniform: V keys take one pass
          const int key = rpart * 32 + (x * 1024 + lane * 16) / bpk;
          if (key < R.nvalid) dma<16>(R.src + x * 1024 + lane * 16, dst + x * 256);
        }
      }
    } else {                                     // scales (2G bytes per key) or labels (1 byte per key)
      const int lead = lead_of((uint32_t)reinterpret_cast<uintptr_t>(R.src));
      const uint8_t* base = R.src - lead;
      const int words = (lead + R.nvalid * bpk + 3) >> 2;
#pragma unroll
      for (int x = 0; x < 3; ++x) {              // at most 3 + 640 bytes: 161 words
        const int wd = x * 64 + lane;
        if (x * 64 < words && wd < words) {
          if (rsel == 1) dma<4>(base + wd * 4, rv ? &sRsV[r][x * 128] : &sRsK[r][x * 128]);
          else dma<4>(base + wd * 4, &sRl[r][rv][x * 256]);
        }
      }
    }
  };
  // (2) centroid gather (labels in ring slot r) into staging slot g: per
  // tensor 16 copies of 4 rows, two per wave; the labels are read first.
  auto cent_gather = [&](const GatherView& G, int r, int g) __attribute__((always_inline)) {
    const int lane = xtid & 63;
    int lab[2][2];
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int x = 0; x < 2; ++x) lab[v][x] = sRl[r][v][G.lead[v] + (xwave * 2 + x) * 4 + (lane >> 4)];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if ((v == 0 && !KFAST) || (v == 1 && !VFAST)) continue;
      const uint16_t* cent = reinterpret_cast<const uint16_t*>(G.cent[v]);
      const int C = v ? vC : kC;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int n = xwave * 2 + x;
        if (n * 4 + (lane >> 4) < G.nvalid)
          dma<16>(cent + min(lab[v][x], C - 1) * kHeadDim + (lane & 15) * 8,
                  v ? &sCentV[g][n * 4 * kHeadDim] : &sCentK[g][n * 4 * kHeadDim]);
      }
    }
  };
  // (3) decode tile j (ring slot r, staging slot g) into LDS buffer b
  auto decode_tile = [&](const DecodeView& D, int j, int r, int g, int b) __attribute__((always_inline)) {
    const int tid = xtid;
    const int nvalid = D.nvalid;
    const int klead = D.lead[0], vlead = D.lead[1];
#pragma unroll
    for (int x = 0; x < kItems; ++x) {          // K: (key, 8 channels) per item
      const int item = tid + x * kThreads;
      const int key = item >> 4, k0 = (item & 15) * 8;
      const bool ok = key < nvalid;
      uint32_t o4[4];
      // keys past nvalid decode stale LDS contents (zero at the start, then
      // earlier tiles' values): finite, and their scores are masked (probability 0)
      if (FRESH && D.fresh) {                    // a fresh-chunk tile: the keys as given, scaled
        if (a.kf.dtype == 2) {                   // dense fp16 rows of a decoded cache, already scaled
          const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.kf.ptr) +
                                                          (int64_t)(D.ftok0 + min(key, nvalid - 1)) * a.kf.stride_token +
                                                          (int64_t)h * a.kf.stride_head + k0);
          o4[0] = w.x; o4[1] = w.y; o4[2] = w.z; o4[3] = w.w;
        } else {
          float v[8];
          fresh_row<8>(a.kf, D.ftok0 + min(key, nvalid - 1), h, k0, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = pack_f16x2(v[2 * e] * ksc, v[2 * e + 1] * ksc);
        }
      } else if constexpr (KM == 1) {
        const uint32_t w = sRcK[r][key * 8 + (k0 >> 4)];
        const uint32_t sb = sRsK[r][klead + (key << kGs) + ((k0 << kGs) >> 7)];   // groups: powers of two
        const uint4 cr = *reinterpret_cast<const uint4*>(&sCentK[g][key * kHeadDim + k0]);
        const uint32_t code16 = (w >> (16 * ((k0 >> 3) & 1))) & 0xFFFFu;
        const uint32_t cw[4] = {cr.x, cr.y, cr.z, cr.w};
        decode_pairs_f16<4>(code16 | (code16 << 14), bf16_bits_to_f32(sb) * ksc, cw, o4);
      } else if constexpr (KM == 2) {
        // item k0 / 8 (= tid % 16) of the mix4 order: one code word, the scales
        // of its (at most two) groups, centroid values already in item order
        const uint32_t w = sRcK[r][key * 16 + (k0 >> 3)];
        const int srow = klead + key * kGn;
        const uint32_t slo = sRsK[r][srow + (int)(mdesc & 0xFFu)], shi = sRsK[r][srow + (int)((mdesc >> 8) & 0xFFu)];
        const uint4 cr = *reinterpret_cast<const uint4*>(&sCentK[g][key * kHeadDim + k0]);
        const uint32_t cw[4] = {cr.x, cr.y, cr.z, cr.w};
        decode_mix4(w, bf16_bits_to_f32(slo) * ksc, bf16_bits_to_f32(shi) * ksc, (int)(mdesc >> 16), cw, o4);
      } else {
        float v[8];
        if (ok && a.kp.n_int4 == 0) decode_uniform<8>(geom(tiles[j].chunk, false), h, tiles[j].token0 + key, k0, v);
        else if (ok) decode_generic<8>(geom(tiles[j].chunk, false), sTabK, h, tiles[j].token0 + key, k0, v);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = pack_f16x2(v[2 * e] * ksc, v[2 * e + 1] * ksc);
      }
      *reinterpret_cast<uint4*>(&sK[b][key][k0]) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
#pragma unroll
    for (int x = 0; x < kItems; ++x) {          // V: (2 keys, 4 channels) per item, channels fastest
      const int item = tid + x * kThreads;
      const int k0 = (item & 31) * 4, kp = item >> 5;
      uint32_t pr[2][2];                         // [key][channel pair] fp16 pairs
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int key = 2 * kp + y;
        const bool ok = key < nvalid;
        if (FRESH && D.fresh) {
          if (a.vf.dtype == 2) {                 // dense fp16 rows, already scaled
            const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.vf.ptr) +
                                                            (int64_t)(D.ftok0 + min(key, nvalid - 1)) * a.vf.stride_token +
                                                            (int64_t)h * a.vf.stride_head + k0);
            pr[y][0] = w.x;
            pr[y][1] = w.y;
          } else {
            float v[4];
            fresh_row<4>(a.vf, D.ftok0 + min(key, nvalid - 1), h, k0, v);
            pr[y][0] = pack_f16x2(v[0] * vsc, v[1] * vsc);
            pr[y][1] = pack_f16x2(v[2] * vsc, v[3] * vsc);
          }
        } else if constexpr (VFAST) {
          const uint32_t w = sRcV[r][key * 8 + (k0 >> 4)];
          const uint32_t sb = sRsV[r][vlead + (key << vGs) + ((k0 << vGs) >> 7)];
          const uint2 cr = *reinterpret_cast<const uint2*>(&sCentV[g][key * kHeadDim + k0]);
          const uint32_t code8 = (w >> (2 * (k0 & 15))) & 0xFFu;   // keys past nvalid: finite, weight 0
          const uint32_t cw[2] = {cr.x, cr.y};
          decode_pairs_f16<2>(code8 | (code8 << 14), bf16_bits_to_f32(sb) * vsc, cw, pr[y]);
        } else {
          float v[4];
          if (ok && a.vp.n_int4 == 0) decode_uniform<4>(geom(tiles[j].chunk, true), h, tiles[j].token0 + key, k0, v);
          else if (ok) decode_generic<4>(geom(tiles[j].chunk, true), sTabV, h, tiles[j].token0 + key, k0, v);
          else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = 0.0f;
          }
          pr[y][0] = pack_f16x2(v[0] * vsc, v[1] * vsc);
          pr[y][1] = pack_f16x2(v[2] * vsc, v[3] * vsc);
        }
      }
      // channel k0 + e gets (key 2kp, key 2kp + 1)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        *reinterpret_cast<uint32_t*>(&sVt[b][k0 + 2 * jj][2 * kp]) = __builtin_amdgcn_perm(pr[1][jj], pr[0][jj], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&sVt[b][k0 + 2 * jj + 1][2 * kp]) = __builtin_amdgcn_perm(pr[1][jj], pr[0][jj], 0x07060302u);
      }
    }
    if (PSAC && tid < kKTile) {
      uint32_t f16w[4] = {0u, 0u, 0u, 0u};
      if (tid < nvalid && !(FRESH && D.fresh)) { // fresh keys carry no correction
        const int rank = a.psac_rank;
        const uint16_t* cpp = reinterpret_cast<const uint16_t*>(m64(j, kFPsac)) + ((int64_t)h * (int)m32(j, kFN) + tid) * rank;
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = e < rank ? bf16_bits_to_f32(cpp[e]) * ksc : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f16w[e] = pack_f16x2(f[2 * e], f[2 * e + 1]);
      }
      *reinterpret_cast<uint4*>(&sKp[b][tid][0]) = make_uint4(f16w[0], f16w[1], f16w[2], f16w[3]);
      *reinterpret_cast<uint4*>(&sKp[b][tid][8]) = make_uint4(f16w[0], f16w[1], f16w[2], f16w[3]);
    }
  };
  // mix4 keys: the queries in the item order of chunk ch's channel permutation
  // (reloaded by each wave when the chunk of its compute tile changes)
  int q_chunk = -1;
  auto load_q_mix = [&](int ch) __attribute__((always_inline)) {
    const int lane = xtid & 63, half = lane >> 5;
    // the fresh chunk's tiles (ch == n_chunks) hold keys in channel order
    const uint8_t* prow = nullptr;
    if (!FRESH || ch < a.n_chunks) {
      const ChunkDecode d = make_decode(a.kp, recs[ch].n, recs[ch].kbase);
      prow = d.base + d.off_perm + (int64_t)h * kHeadDim;
    }
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q.ptr) + (int64_t)(qok ? qrow : 0) * a.q.stride_token +
                         (int64_t)h * a.q.stride_head;
    // per k-step: the eight item positions from LDS in one read, then eight
    // independent order-byte loads, then eight independent query loads (the
    // query row is clamped to a valid one, so no load is predicated): two
    // memory round trips per k-step
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint2 rr = *reinterpret_cast<const uint2*>(&sRho[s * 16 + half * 8]);
      const uint32_t r2[2] = {rr.x, rr.y};
      uint32_t k8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t P = (r2[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        if constexpr (FRESH) k8[e] = prow ? prow[P] : (uint32_t)(s * 16 + half * 8 + e);
        else k8[e] = prow[P];
      }
      uint32_t q8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q8[e] = qp[k8[e] & (kHeadDim - 1)];
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qok ? bf16_bits_to_f32(q8[e]) : 0.0f;
        hv[e] = (_Float16)__builtin_amdgcn_fmed3f(v * qsc, -kF16Max, kF16Max);
      }
      qh[s] = hv;
    }
  };
  // (4) this wave's 32 queries against tile j in LDS buffer b
  auto compute_tile = [&](int nvalid, int kstart, int b, int chunk) __attribute__((always_inline)) {
    const int lane = xtid & 63, col = lane & 31, half = lane >> 5;
    if (!wave_active) return;
    if constexpr (KM == 2) {
      if (chunk != q_chunk) {                   // wave-uniform
        load_q_mix(chunk);
        q_chunk = chunk;
      }
    }
    if (a.causal && !LOGITS && kstart >= vis_end(wq_last)) return;     // wholly invisible to this wave
    const bool need_mask = nvalid < kKTile || (a.causal && kstart + kKTile > vis_end(wq_first));
    // S^T = K_hat Q^T, both 32-key halves interleaved (fp16 operands, fp32 accumulation)
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    // K fragments of step s + 1 are read from LDS while step s multiplies
    auto kfrag = [&](int s, int kb) __attribute__((always_inline)) {
      return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(&sK[b][kb * 32 + col][s * 16 + half * 8]));
    };
    f16x8 knext[2] = {kfrag(0, 0), kfrag(0, 1)};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f16x8 kf[2] = {knext[0], knext[1]};
      if (s + 1 < 8) {
        knext[0] = kfrag(s + 1, 0);
        knext[1] = kfrag(s + 1, 1);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[kb], qh[s], acc[kb], 0, 0, 0);
        if constexpr (QF32) acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[kb], ql[QF32 ? s : 0], acc[kb], 0, 0, 0);
      }
    }
    // instruction order of the loop above: the first step's two LDS reads, then
    // per step the next step's two reads ahead of this step's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, QF32 ? 4 : 2, 0);
    }
    if constexpr (PSAC) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f16x8 kpf = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(&sKp[b][kb * 32 + col][half * 8]));
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kpf, qpsac, acc[kb], 0, 0, 0);
      }
    }
    float sv[32];                                // key kb*32 + (r/4)*8 + half*4 + r%4 for sv[kb*16 + r]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[kb * 16 + r] = acc[kb][r];
    if (need_mask || LOGITS) {
      // key kl of element i is kc(i) + half*4; it is visible iff kl < nvalid and
      // (causal modes) kstart + kl < vis_end(qrow), i.e. iff kc(i) < lim.  The
      // select is done with integer bit operations, not per-element compare masks.
      int lim = nvalid;
      if (a.causal) lim = min(lim, vis_end(qrow) - kstart);
      lim -= half * 4;
      // opaque here, so the 32 differences below are formed only in masked
      // tiles (hoisted, they cost 32 VALU and 31 VGPRs in every tile)
      asm volatile("" : "+v"(lim));
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int kc = (i >> 4) * 32 + ((i & 15) >> 2) * 8 + (i & 3);
        uint32_t masked;                                          // all ones when hidden
        asm("v_ashrrev_i32 %0, 31, %1" : "=v"(masked) : "v"(lim - 1 - kc));   // kept arithmetic (no compare mask)
        if (LOGITS) {
          const int kl = kc + half * 4;
          if (qok && kl < nvalid)
            a.logits[((int64_t)h * a.Nq + qrow) * a.Nk + (int64_t)(kstart + kl)] = masked ? -INFINITY : sv[i] * sfull;
        }
        sv[i] = __uint_as_float((__float_as_uint(sv[i]) & ~masked) | (0xFF800000u & masked));
      }
    }
    float mloc = sv[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mloc = fmaxf(mloc, sv[i]);
    mloc = max_with_other_half(mloc);
    const float m_cand = mloc * c2;                             // c2 > 0
    // lazy rescaling: keep the running max unless it grows by more than 8 (p <= 2^8)
    const bool grow = m_cand > m_run + 8.0f;
    float alpha = 1.0f;
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, m_cand);
      alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    const float mneg = m_run == -INFINITY ? 0.0f : -m_run;
    // hardware exp2 (v_exp_f32): arguments are <= 8 here; results below the
    // fp32 normal range flush to zero, which a probability can afford.  The sum
    // runs over the fp16-rounded probabilities that enter P V.
    uint32_t pw[4][4];                           // [16-key step][pair]
    float psum = 0.0f;
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      f16x2 pp;
      pp[0] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, mneg));
      pp[1] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[i + 1], c2, mneg));
      psum = __builtin_amdgcn_fdot2(pp, ones, psum, false);
      pw[i >> 3][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, pp);
    }
    l_run = l_run * alpha + psum;
    // O^T += V_hat^T P^T: A = V_hat^T (row = channel, k = key slot), B = P^T
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kbase = st * 16 + half * 4;
      f16x8 vf[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int drow = db * 32 + col;
        const uint32_t* vrow = reinterpret_cast<const uint32_t*>(&sVt[b][drow][kbase]);   // 4-byte aligned
        vf[db] = __builtin_bit_cast(f16x8, make_uint4(vrow[0], vrow[1], vrow[4], vrow[5]));
      }
      const f16x8 pfrag = __builtin_bit_cast(f16x8, make_uint4(pw[st][0], pw[st][1], pw[st][2], pw[st][3]));
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[db], pfrag, o[db], 0, 0, 0);
    }
  };
  // generic decode tables follow the chunk of the tile being decoded
  int gen_chunk = -1;
  auto tables_for = [&](int j) __attribute__((always_inline)) {
    if constexpr (!KFAST || !VFAST) {
      if (FRESH && j >= a.n_cache_tiles) return; // fresh-chunk tiles need no tables
      const int chunk = tiles[j].chunk;
      if (chunk != gen_chunk) {
        __syncthreads();
        if constexpr (!KFAST) build_tab(geom(chunk, false), h, sTabK);
        if constexpr (!VFAST) build_tab(geom(chunk, true), h, sTabV);
        __syncthreads();
        gen_chunk = chunk;
      }
    }
  };

  // ---- prologue: tiles t_begin .. t_begin+2 raw, t_begin .. t_begin+1 gathered, t_begin decoded ----
  if constexpr (KFAST || VFAST) {
    // The fast decode reads the staging slots for every key of a tile, also
    // past its end, where no copy lands: zeroed here, they only ever hold
    // finite values (zeros or earlier tiles' scales and centroid rows), and
    // the barrier below orders these writes before the first copies.
    uint4* ck = reinterpret_cast<uint4*>(&sCentK[0][0]);
    uint4* cv = reinterpret_cast<uint4*>(&sCentV[0][0]);
    for (int i = tid; i < (int)(sizeof(sCentK) / 16); i += kThreads) {
      ck[i] = make_uint4(0u, 0u, 0u, 0u);
      cv[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t* rsk = reinterpret_cast<uint32_t*>(&sRsK[0][0]);
    for (int i = tid; i < (int)(sizeof(sRsK) / 4); i += kThreads) rsk[i] = 0u;
    uint32_t* rsv = reinterpret_cast<uint32_t*>(&sRsV[0][0]);
    for (int i = tid; i < (int)(sizeof(sRsV) / 4); i += kThreads) rsv[i] = 0u;
  }
  if constexpr (KM == 2) {
    if (tid < kHeadDim) sRho[tid] = a.mixp->rho[tid];
  }
  const int r0 = t_begin % kRing;
  if (xwave == 0) {
#pragma unroll 1
    for (int k = 0; k < 5 && t_begin + k < t_end; ++k) meta_copy(t_begin + k);
  }
  wait_dma();
  __syncthreads();
#pragma unroll 1
  for (int k = 0; k < 3 && t_begin + k < t_end; ++k)
    if (!FRESH || t_begin + k < a.n_cache_tiles) raw_copy(raw_view(t_begin + k, true), (r0 + k) % kRing);
  wait_dma();
  __syncthreads();
  if (!FRESH || t_begin < a.n_cache_tiles) cent_gather(gather_view(t_begin, true), r0, t_begin & 1);
  if (t_begin + 1 < t_end && (!FRESH || t_begin + 1 < a.n_cache_tiles))
    cent_gather(gather_view(t_begin + 1, true), (r0 + 1) % kRing, (t_begin + 1) & 1);
  wait_dma();
  __syncthreads();
  tables_for(t_begin);
  decode_tile(decode_view(t_begin, true), t_begin, r0, t_begin & 1, t_begin & 1);
  __syncthreads();

  int ring = r0;                                 // ring slot of tile ti
#pragma unroll 1
  for (int ti = t_begin; ti < t_end; ++ti) {
    xtid = tid;
    xwave = wave;
    // the lean fast-decode variants keep their lane addresses in registers
    // (101 instead of 204 VALU of per-step set-up, no spills); the others would
    // spill them, so there the thread index is made opaque too
    constexpr bool kLaneAddrKept = !QF32 && KM != 0 && VFAST && !LOGITS && !PSAC && !FRESH;
    if constexpr (kLaneAddrKept) asm volatile("" : "+s"(xwave));
    else asm volatile("" : "+v"(xtid), "+s"(xwave));
    const int r3 = ring;                         // (ti + 3) % 3
    const int r1 = ring + 1 == kRing ? 0 : ring + 1;
    const int r2 = r1 + 1 == kRing ? 0 : r1 + 1;
    const bool has1 = ti + 1 < t_end, has2 = ti + 2 < t_end, has3 = ti + 3 < t_end;
    // this step's tile-record fields, loaded up front (indexes clamped to
    // real tiles; the view of a missing tile has nvalid = 0 and is not used)
    const int j1 = has1 ? ti + 1 : ti, j2 = has2 ? ti + 2 : ti, j3 = has3 ? ti + 3 : ti;
    // all metadata words of this step, read from LDS as one batch
    const RawRole q = raw_role();
    const uint32_t* M0 = sMeta[ti % kMetaSlots];
    const uint32_t* M1 = sMeta[j1 % kMetaSlots];
    const uint32_t* M2 = sMeta[j2 % kMetaSlots];
    const uint32_t* M3 = sMeta[j3 % kMetaSlots];
    const int fs = kFSrc + (q.rv * 3 + q.rsel) * 2;
    uint32_t w[19] = {M0[kFNvalid], M0[kFKstart],
                      M1[kFNvalid], M1[kFN], M1[kFSrc + 2], M1[kFSrc + 8],
                      M2[kFNvalid], M2[kFN], M2[kFCent], M2[kFCent + 1], M2[kFCent + 2], M2[kFCent + 3],
                      M2[kFSrc + 4], M2[kFSrc + 10],
                      M3[kFNvalid], M3[kFN], M3[fs], M3[fs + 1], KM == 2 ? M0[kFChunk] : 0u};
#pragma unroll
    for (int k = 0; k < 19; ++k) w[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)w[k]);
    const int nv0 = (int)w[0], ks0 = (int)w[1], ch0 = (int)w[18];
    DecodeView DV;
    {
      const uint32_t hrow = (uint32_t)h * w[3];
      DV.lead[0] = lead_of(w[4] + hrow * (uint32_t)(2 * kGn)) >> 1;   // K scales
      DV.lead[1] = lead_of(w[5] + (hrow << (vGs + 1))) >> 1;     // V scales
      DV.nvalid = has1 ? (int)w[2] : 0;
      DV.fresh = FRESH && j1 >= a.n_cache_tiles;
      DV.ftok0 = FRESH ? (j1 - a.n_cache_tiles) * kKTile : 0;
    }
    GatherView GV;
    {
      const uint32_t hrow = (uint32_t)h * w[7];
      GV.cent[0] = reinterpret_cast<const uint8_t*>(((uint64_t)w[9] << 32) | w[8]) + (int64_t)h * kC * kHeadDim * 2;
      GV.cent[1] = reinterpret_cast<const uint8_t*>(((uint64_t)w[11] << 32) | w[10]) + (int64_t)h * vC * kHeadDim * 2;
      GV.lead[0] = lead_of(w[12] + hrow);                         // K labels
      GV.lead[1] = lead_of(w[13] + hrow);                         // V labels
      GV.nvalid = has2 ? (int)w[6] : 0;
    }
    RawView RV;
    {
      const int64_t hrow = (int64_t)h * (int)w[15];
      RV.src = reinterpret_cast<const uint8_t*>(((uint64_t)w[17] << 32) | w[16]) + hrow * q.bpk + (q.rpart == 1 ? 32 * q.bpk : 0);
      RV.nvalid = has3 ? (int)w[14] : 0;
    }
    if (has1) tables_for(j1);
    // (1) raw copy of tile i+3 and (2) centroid gather of tile i+2 are issued
    // after this wave's decode (its reads of the copy targets would otherwise
    // wait for them) and before its compute, which reads other LDS objects.
    auto issue = [&]() __attribute__((always_inline)) {
      if (has2 && (!FRESH || j2 < a.n_cache_tiles)) cent_gather(GV, r2, ti & 1);
      if (has3 && (!FRESH || j3 < a.n_cache_tiles)) raw_copy(RV, r3);
      if (xwave == 0 && ti + 5 < t_end) meta_copy(ti + 5);   // slot of tile i+5: read from step i+2 on
    };
#pragma unroll 1
    for (int ph = 0; ph < 2; ++ph) {
      if (ph == grp) {
        if (grp == 0) issue();
        compute_tile(nv0, ks0, ti & 1, ch0);                                // (4) tile i
      } else {
        if (has1) decode_tile(DV, j1, r1, (ti + 1) & 1, (ti + 1) & 1);      // (3) tile i+1
        if (grp == 1) issue();
      }
    }
    wait_dma();
    __syncthreads();
    ring = r1;
  }

  // ---- epilogue ----
  // The output arguments are read here, through an opaque pointer to the
  // kernel arguments, so that they are not held in registers during the loop.
  cargs_ptr E = (cargs_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(E));
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qok) return;
  if (E->n_split_total == 1) {
    const float inv = l_tot > 0.0f ? pow2(rx.ev) / l_tot : 0.0f;
    float* orow = E->out + (int64_t)qrow * E->out_stride_token + (int64_t)h * E->out_stride_head;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        *reinterpret_cast<float4*>(orow + d0) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      }
  } else {
    const int ps = E->split_base + split;
    float* prow = E->part_o + (((int64_t)ps * E->H + h) * E->Nq + qrow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        *reinterpret_cast<float4*>(prow + d0) = make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
      }
    if (half == 0) {
      float* ml = E->part_ml + (((int64_t)ps * E->H + h) * E->Nq + qrow) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Merge the splits: thread = (head, query, 4 channels).
__global__ __launch_bounds__(256) void k_merge(AttendArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.H * a.Nq * (kHeadDim / 4);
  if (gid >= total) return;
  const int d0 = (int)(gid % (kHeadDim / 4)) * 4;
  const int64_t hq = gid / (kHeadDim / 4);
  const int qrow = (int)(hq % a.Nq), h = (int)(hq / a.Nq);
  float mmax = -INFINITY;
  for (int s = 0; s < a.n_split_total; ++s)
    mmax = fmaxf(mmax, a.part_ml[(((int64_t)s * a.H + h) * a.Nq + qrow) * 2]);
  float4 acc = make_float4(0, 0, 0, 0);
  float lsum = 0.0f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < a.n_split_total; ++s) {
      const int64_t r = ((int64_t)s * a.H + h) * a.Nq + qrow;
      const float ms = a.part_ml[r * 2];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - mmax);
      lsum += wgt * a.part_ml[r * 2 + 1];
      const float4 v = *reinterpret_cast<const float4*>(a.part_o + r * kHeadDim + d0);
      acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
    }
  }
  const int ev = range_exps(a.range, a.kp, a.vp, a.psac_rank > 0).ev;
  const float inv = lsum > 0.0f ? pow2(ev) / lsum : 0.0f;
  float* orow = a.out + (int64_t)qrow * a.out_stride_token + (int64_t)h * a.out_stride_head + d0;
  *reinterpret_cast<float4*>(orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// qU[h][i][b] = sum_k q_ik U[h][k][b] (float64 accumulation, rounded to fp32);
// the largest |qU| of the call goes to the range record.
template <bool QF32>
__global__ __launch_bounds__(256) void k_qu(TensorView q, int H, int Nq, int r, const float* __restrict__ U,
                                            float* __restrict__ qu, uint32_t* __restrict__ range) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float mx = 0.0f;
  if (gid < (int64_t)H * Nq) {
    const int i = (int)(gid % Nq), h = (int)(gid / Nq);
    double acc[kMaxRank];
#pragma unroll
    for (int b = 0; b < kMaxRank; ++b) acc[b] = 0.0;
    const int64_t base = (int64_t)i * q.stride_token + (int64_t)h * q.stride_head;
    for (int k = 0; k < kHeadDim; ++k) {
      float qv;
      if constexpr (QF32) qv = reinterpret_cast<const float*>(q.ptr)[base + k];
      else qv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q.ptr)[base + k]);
#pragma unroll
      for (int b = 0; b < kMaxRank; ++b)
        if (b < r) acc[b] += (double)qv * (double)U[((int64_t)h * kHeadDim + k) * r + b];
    }
#pragma unroll
    for (int b = 0; b < kMaxRank; ++b) {
      const float v = b < r ? (float)acc[b] : 0.0f;
      qu[gid * kMaxRank + b] = v;
      mx = fmaxf(mx, fabsf(v));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) atomicMax(range + kRgQU, __float_as_uint(mx));
}

// TileRec of every tile: the chunk holding it is the last one whose first tile is <= j.
__global__ __launch_bounds__(256) void k_tile_table(const ChunkRec* __restrict__ recs, int n_chunks, int n_tiles,
                                                    int n_cache_tiles, int n_fresh, int64_t fresh_start,
                                                    TokenBytes tb, int H, int kC, int vC, const uint16_t* k16,
                                                    const uint16_t* v16, TileRec* __restrict__ tiles) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_tiles) return;
  if (j >= n_cache_tiles) {                      // a tile of the fresh chunk: geometry only
    TileRec t{};
    const int token0 = (j - n_cache_tiles) * kKTile;
    t.n = n_fresh;
    t.nvalid = min(kKTile, n_fresh - token0);
    t.kstart = (int)fresh_start + token0;
    t.token0 = token0;
    t.chunk = n_chunks;
    tiles[j] = t;
    return;
  }
  int lo = 0, hi = n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (recs[mid].tile_start <= j) lo = mid; else hi = mid - 1;
  }
  const ChunkRec& c = recs[lo];
  const int token0 = (j - c.tile_start) * kKTile;
  TileRec t;
  t.src[0][0] = (c.krep ? c.krep : c.kcodes) + (int64_t)token0 * tb.kcodes;
  t.src[1][0] = c.vcodes + (int64_t)token0 * tb.vcodes;
  t.src[0][1] = c.kscales + (int64_t)token0 * tb.kscales;
  t.src[1][1] = c.vscales + (int64_t)token0 * tb.vscales;
  t.src[0][2] = c.klabels + token0;
  t.src[1][2] = c.vlabels + token0;
  t.cent[0] = k16 ? reinterpret_cast<const uint8_t*>(k16 + (int64_t)lo * H * kC * kHeadDim) : c.kcent;
  t.cent[1] = v16 ? reinterpret_cast<const uint8_t*>(v16 + (int64_t)lo * H * vC * kHeadDim) : c.vcent;
  t.kpsac = c.kpsac + (int64_t)token0 * tb.kpsac;
  t.n = c.n;
  t.nvalid = min(kKTile, c.n - token0);
  t.kstart = (int)c.token_start + token0;
  t.token0 = token0;
  t.chunk = lo;
  t.pad = 0;
  tiles[j] = t;
}

// Thread: 8 channels of one centroid row; blockIdx.y: 0 keys, 1 values.  The
// rows are scaled by the tensor's range exponent (exact) and rounded to fp16.
__global__ __launch_bounds__(256) void k_centroids_f16(const ChunkRec* __restrict__ recs, int n_chunks, LayoutParams kp,
                                                       LayoutParams vp, const uint32_t* __restrict__ range,
                                                       const MixOrder* __restrict__ kmix,
                                                       uint16_t* __restrict__ k16, uint16_t* __restrict__ v16) {
  const bool v = blockIdx.y == 1;
  uint16_t* dst = v ? v16 : k16;
  const int C = v ? vp.C : kp.C, H = kp.H;
  if (!dst) return;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_chunk = (int64_t)H * C * (kHeadDim / 8);
  if (gid >= per_chunk * n_chunks) return;
  const RangeExps rx = range_exps(range, kp, vp, kp.psac_rank > 0);
  const float sc = pow2(-(v ? rx.ev : rx.ek));
  const int chunk = (int)(gid / per_chunk);
  const int64_t e = (gid % per_chunk) * 8;      // element within the chunk's [H][C][128] table
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v ? recs[chunk].vcent : recs[chunk].kcent);
  uint32_t w4[4];
  if (!v && kmix) {
    // mix4 keys: the row in item order, through the chunk's channel permutation
    const ChunkDecode d = make_decode(kp, recs[chunk].n, recs[chunk].kbase);
    const int64_t row = e >> 7;                                    // h * C + j
    const uint8_t* prow = d.base + d.off_perm + (row / C) * kHeadDim;
    const int r0 = (int)(e & (kHeadDim - 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = src[row * kHeadDim + (prow[kmix->rho[r0 + 2 * k]] & (kHeadDim - 1))];
      const uint32_t hi = src[row * kHeadDim + (prow[kmix->rho[r0 + 2 * k + 1]] & (kHeadDim - 1))];
      w4[k] = lo | (hi << 16);
    }
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(src + e);
    w4[0] = w.x; w4[1] = w.y; w4[2] = w.z; w4[3] = w.w;
  }
  uint32_t o4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f16x2 r;
    r[0] = (_Float16)__builtin_amdgcn_fmed3f(__uint_as_float(w4[k] << 16) * sc, -kF16Max, kF16Max);
    r[1] = (_Float16)__builtin_amdgcn_fmed3f(__uint_as_float(w4[k] & 0xFFFF0000u) * sc, -kF16Max, kF16Max);
    o4[k] = __builtin_bit_cast(uint32_t, r);
  }
  *reinterpret_cast<uint4*>(dst + chunk * per_chunk * 8 + e) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
}

// Largest bf16 magnitude (as float32 bits) of n values at p: this thread's
// share of a grid-stride pass over uint4 words, then the scalar tail.
__device__ __forceinline__ uint32_t bf16_absmax(const uint16_t* p, int64_t n, int64_t start, int64_t step) {
  uint32_t m = 0;
  const int64_t nv = n / 8;
  const uint4* p4 = reinterpret_cast<const uint4*>(p);
  for (int64_t i = start; i < nv; i += step) {
    const uint4 w = p4[i];
    const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(w4[k] & 0x7FFFu, (w4[k] >> 16) & 0x7FFFu));
  }
  for (int64_t i = nv * 8 + start; i < n; i += step) m = max(m, (uint32_t)p[i] & 0x7FFFu);
  return m << 16;
}

// Largest |x| (float32 bits) of a strided [rows / H][H][128] tensor: this
// thread's share of a grid-stride pass over its uint4 words.
__device__ __forceinline__ uint32_t tensor_absmax(const TensorView& t, int H, int64_t rows, int64_t start, int64_t step) {
  uint32_t m = 0;
  const int per_row = t.dtype == 0 ? 32 : 16;    // uint4 words per row of 128 values
  for (int64_t i = start; i < rows * per_row; i += step) {
    const int64_t row = i / per_row;
    const int64_t off = (row / H) * t.stride_token + (row % H) * t.stride_head;
    if (t.dtype == 0) {
      const uint4 w = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(t.ptr) + off)[i % per_row];
      m = max(m, max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu)));
    } else {
      const uint4 w = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(t.ptr) + off)[i % per_row];
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, max(w4[k] & 0x7FFFu, (w4[k] >> 16) & 0x7FFFu) << 16);
    }
  }
  return m;
}

// Range scan.  blockIdx.y = 2 chunk + tensor for the chunks' stored scales,
// centroids (every stage) and PSAC coefficients; blockIdx.y = 2 n_chunks + 0,
// 1, 2 for the queries, the fresh keys and the fresh values.  Each block reduces
// its share and adds it with one atomic max per slot.
__global__ __launch_bounds__(256) void k_range_scan(const ChunkRec* __restrict__ recs, int n_chunks, LayoutParams kp,
                                                    LayoutParams vp, TensorView q, int Nq, TensorView kf,
                                                    TensorView vf, int n_fresh, uint32_t* __restrict__ range) {
  __shared__ uint32_t red[3][4];
  const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  uint32_t m[3] = {0u, 0u, 0u};                  // scale, centroid, coefficient (or query)
  const int y = blockIdx.y;
  if (y < 2 * n_chunks) {
    const bool v = y & 1;
    const ChunkRec& c = recs[y >> 1];
    const LayoutParams& p = v ? vp : kp;
    const ChunkDecode d = make_decode(p, c.n, v ? c.vbase : c.kbase);
    for (int l = 0; l < d.n_stages; ++l) {
      m[0] = max(m[0], bf16_absmax(reinterpret_cast<const uint16_t*>(d.base + d.off_scales + d.stage_scales * l),
                                   (int64_t)d.H * d.N * d.groups, start, step));
      m[1] = max(m[1], bf16_absmax(reinterpret_cast<const uint16_t*>(d.base + d.off_centroids + d.stage_centroids * l),
                                   (int64_t)d.H * d.C * kHeadDim, start, step));
    }
    if (d.psac_rank > 0)
      m[2] = bf16_absmax(reinterpret_cast<const uint16_t*>(d.base + d.off_psac), (int64_t)d.H * d.N * d.psac_rank,
                         start, step);
  } else if (y == 2 * n_chunks) {
    m[2] = tensor_absmax(q, kp.H, (int64_t)Nq * kp.H, start, step);
  } else if (n_fresh > 0) {
    m[2] = tensor_absmax(y == 2 * n_chunks + 1 ? kf : vf, kp.H, (int64_t)n_fresh * kp.H, start, step);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < 3; ++k) red[k][wave] = m[k];
  __syncthreads();
  if (threadIdx.x < 3) {
    const int k = threadIdx.x;
    const uint32_t r = max(max(red[k][0], red[k][1]), max(red[k][2], red[k][3]));
    int slot;
    if (y < 2 * n_chunks) slot = k == 2 ? kRgCoef : ((y & 1) ? (k == 0 ? kRgVScale : kRgVCent) : (k == 0 ? kRgKScale : kRgKCent));
    else slot = k != 2 ? -1 : y == 2 * n_chunks ? kRgQ : y == 2 * n_chunks + 1 ? kRgKFresh : kRgVFresh;
    if (slot >= 0 && r != 0u) atomicMax(range + slot, r);
  }
}

// Caches that take the generic decode (several stages, INT4, groups that are
// not multiples of 32): every (chunk, head) is decoded once per call into
// dense fp16 rows [Nk][H][128] of K and of V, with the tile decode's own
// arithmetic and operand scaling (decode_uniform or decode_generic, then
// fp16(x * 2^-e)), so attending over them as fresh-chunk tiles gives the
// attention of the generic decode.  Block (64-token block, head, chunk).
__global__ __launch_bounds__(256) void k_dense_decode(const ChunkRec* __restrict__ recs, LayoutParams kp,
                                                      LayoutParams vp, const uint32_t* __restrict__ range,
                                                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  __shared__ ChannelCode sTab[2][kHeadDim];
  const ChunkRec& c = recs[blockIdx.z];
  const int h = blockIdx.y, H = gridDim.y, t0 = blockIdx.x * 64;
  if (t0 >= c.n) return;                         // the whole block
  const RangeExps rx = range_exps((crange_ptr)range, kp, vp, false);
  const float sc[2] = {pow2(-rx.ek), pow2(-rx.ev)};
  const ChunkDecode dd[2] = {make_decode(kp, c.n, c.kbase), make_decode(vp, c.n, c.vbase)};
  if (kp.n_int4 > 0) build_tab(dd[0], h, sTab[0]);
  if (vp.n_int4 > 0) build_tab(dd[1], h, sTab[1]);
  __syncthreads();
  const int nt = min(64, c.n - t0);
  for (int item = threadIdx.x; item < 2 * 64 * 16; item += blockDim.x) {   // (tensor, token, 8 channels)
    const int v = item >= 64 * 16, r = item - v * 64 * 16;
    const int key = r >> 4, k0 = (r & 15) * 8;
    if (key >= nt) continue;
    float x[8];
    if ((v ? vp : kp).n_int4 == 0) decode_uniform<8>(dd[v], h, t0 + key, k0, x);
    else decode_generic<8>(dd[v], sTab[v], h, t0 + key, k0, x);
    uint32_t o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = pack_f16x2(x[2 * e] * sc[v], x[2 * e + 1] * sc[v]);
    uint16_t* dst = (v ? dv : dk) + ((int64_t)(c.token_start + t0 + key) * H + h) * kHeadDim + k0;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
}

__global__ void k_upload(ChunkBatch b, ChunkRec* __restrict__ dst, uint32_t* __restrict__ range, MixOrder mix,
                         MixOrder* __restrict__ mix_dst) {
  const int i = threadIdx.x;
  if (i < b.count) dst[b.first + i] = b.rec[i];
  if (b.first == 0 && i < kRangeWords) range[i] = 0u;
  if (b.first == 0 && mix_dst && i == 0) *mix_dst = mix;
}

// mix4 codes: a block takes 256 consecutive (head, token) rows of chunk
// blockIdx.y (one contiguous run of code words, staged in LDS); thread =
// (row, item) writes the item's word, 16 rows per pass: u' = q + 8 of position
// 2j at nibble slot j and of position 2j + 1 at slot j + 4.  (Sixteen rows per
// block made the launch dispatch-bound: 900,000 blocks for the one-minute cache.)
constexpr int kRepackRows = 256;        // token-heads per workgroup (16 per pass of the 256 threads)
constexpr int kRepackMaxWords = 17;   // 4-bit words + 2-bit words of a mixed row (n_int4 = 127)
__global__ __launch_bounds__(256) void k_repack_mix(const ChunkRec* __restrict__ recs, LayoutParams kp,
                                                    const MixOrder* __restrict__ mix) {
  __shared__ uint8_t rho[kHeadDim];
  __shared__ uint32_t sw[kRepackRows * kRepackMaxWords];
  const ChunkRec& c = recs[blockIdx.y];
  const int64_t rows = (int64_t)kp.H * c.n;
  const int64_t r0 = (int64_t)blockIdx.x * kRepackRows;
  if (r0 >= rows) return;                        // the whole block
  const ChunkDecode d = make_decode(kp, c.n, c.kbase);
  const int W = min(d.words, kRepackMaxWords), n4 = d.n_int4, w4 = d.int4_words;
  const int nrows = (int)min<int64_t>(kRepackRows, rows - r0);
  // the block's rows are one contiguous run of nrows * words code words
  const uint32_t* src = reinterpret_cast<const uint32_t*>(d.base + d.off_codes) + r0 * d.words;
  if (W == d.words) {                            // always for a valid layout: one contiguous copy
#pragma unroll 4
    for (int i = threadIdx.x; i < nrows * W; i += blockDim.x) sw[i] = src[i];
  } else {
    for (int i = threadIdx.x; i < nrows * W; i += blockDim.x) sw[i] = src[(i / W) * d.words + i % W];
  }
  if (threadIdx.x < kHeadDim) rho[threadIdx.x] = mix->rho[threadIdx.x];
  __syncthreads();
  // this thread's output word `it` is the same for every row: its eight
  // nibbles' source word, bit offset, width and offset (u' = q + 8: a 4-bit
  // code as stored, a 2-bit code + 6) are fixed before the row loop
  const int it = threadIdx.x & 15;
  int src_w[8];
  uint32_t src_sh[8], src_bw[8], src_ad[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p = rho[it * 8 + t];
    const int pb = p - n4;
    const bool b4 = p < n4;
    src_w[t] = b4 ? min(p >> 3, W - 1) : min(w4 + (pb >> 4), W - 1);
    src_sh[t] = b4 ? 4u * (uint32_t)(p & 7) : 2u * (uint32_t)(pb & 15);
    src_bw[t] = b4 ? 4u : 2u;
    src_ad[t] = b4 ? 0u : 6u;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(c.krep)) + r0 * 16;
  for (int tr = threadIdx.x >> 4; tr < nrows; tr += 16) {   // thread (row, 4-byte output word)
    const uint32_t* rw = sw + tr * W;
    uint32_t acc = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc |= (__builtin_amdgcn_ubfe(rw[src_w[t]], src_sh[t], src_bw[t]) + src_ad[t]) << (4 * ((t >> 1) + 4 * (t & 1)));
    dst[tr * 16 + it] = acc;
  }
}

}  // namespace

hipError_t launch_upload_chunks(const ChunkBatch& b, ChunkRec* dst, uint32_t* range, const MixOrder& mix,
                                MixOrder* mix_dst, hipStream_t s) {
  TimedLaunch tl_("k_upload", s);
  static_assert(kRangeWords <= kChunkBatch, "the upload's threads clear the range record");
  hipLaunchKernelGGL(k_upload, dim3(1), dim3(kChunkBatch), 0, s, b, dst, range, mix, mix_dst);
  return hipGetLastError();
}

hipError_t launch_repack_mix(const ChunkRec* recs, int n_chunks, int max_tokens, const LayoutParams& kp,
                             const MixOrder* mix, hipStream_t s) {
  if (n_chunks <= 0 || max_tokens <= 0) return hipSuccess;
  TimedLaunch tl_("k_repack_mix", s);
  const int64_t per = (int64_t)kp.H * max_tokens;
  hipLaunchKernelGGL(k_repack_mix, dim3((unsigned)((per + kRepackRows - 1) / kRepackRows), (unsigned)n_chunks), dim3(256),
                     0, s, recs, kp, mix);
  return hipGetLastError();
}


hipError_t launch_range_scan(const ChunkRec* recs, int n_chunks, const LayoutParams& kp, const LayoutParams& vp,
                             const TensorView& q, int Nq, const TensorView& kf, const TensorView& vf, int n_fresh,
                             uint32_t* range, hipStream_t s) {
  TimedLaunch tl_("k_range_scan", s);
  const int ys = 2 * n_chunks + 3;
  const int bx = std::max(1, std::min(64, 2048 / ys));
  hipLaunchKernelGGL(k_range_scan, dim3((unsigned)bx, (unsigned)ys), dim3(256), 0, s, recs, n_chunks, kp, vp, q, Nq, kf,
                     vf, n_fresh, range);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const ChunkRec* recs, int n_chunks, int max_n, int H, const LayoutParams& kp,
                               const LayoutParams& vp, const uint32_t* range, uint16_t* dk, uint16_t* dv,
                               hipStream_t s) {
  TimedLaunch tl_("k_dense_decode", s);
  if (n_chunks <= 0 || max_n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dense_decode, dim3((unsigned)((max_n + 63) / 64), (unsigned)H, (unsigned)n_chunks), dim3(256), 0,
                     s, recs, kp, vp, range, dk, dv);
  return hipGetLastError();
}

hipError_t launch_centroids_f16(const ChunkRec* recs, int n_chunks, const LayoutParams& kp, const LayoutParams& vp,
                                const uint32_t* range, const MixOrder* kmix, uint16_t* k16, uint16_t* v16,
                                hipStream_t s) {
  TimedLaunch tl_("k_centroids_f16", s);
  if ((!k16 && !v16) || n_chunks <= 0) return hipSuccess;
  const int64_t per = (int64_t)kp.H * std::max(k16 ? kp.C : 0, v16 ? vp.C : 0) * (kHeadDim / 8) * n_chunks;
  hipLaunchKernelGGL(k_centroids_f16, dim3((unsigned)((per + 255) / 256), 2), dim3(256), 0, s, recs, n_chunks, kp, vp,
                     range, kmix, k16, v16);
  return hipGetLastError();
}

hipError_t launch_tile_table(const ChunkRec* recs, int n_chunks, int n_tiles, int n_cache_tiles, int n_fresh,
                             int64_t fresh_start, TokenBytes tb, int H, int kC, int vC, const uint16_t* k16,
                             const uint16_t* v16, TileRec* tiles, hipStream_t s) {
  TimedLaunch tl_("k_tile_table", s);
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tile_table, dim3((unsigned)((n_tiles + 255) / 256)), dim3(256), 0, s, recs, n_chunks, n_tiles,
                     n_cache_tiles, n_fresh, fresh_start, tb, H, kC, vC, k16, v16, tiles);
  return hipGetLastError();
}

template <int F>
void launch_attend_flags(const AttendArgs& a, dim3 grid, hipStream_t s) {
  constexpr int KM = (F & 32) ? 2 : (F & 2) ? 1 : 0;
  hipLaunchKernelGGL((k_attend<(F & 1) != 0, KM, (F & 4) != 0, (F & 8) != 0, (F & 16) != 0, (F & 64) != 0>), grid,
                     dim3(kThreads), 0, s, a);
}
// flags: 1 fp32 queries, 2 K INT2 fast path, 4 V fast path, 8 debug logits,
// 16 PSAC, 32 K mix4 path (only with bf16 queries and no PSAC), 64 a fresh
// chunk (only with bf16 queries)
template <int... F>
void launch_attend_variant(int flags, const AttendArgs& a, dim3 grid, hipStream_t s, std::integer_sequence<int, F...>) {
  ((flags == F ? launch_attend_flags<F>(a, grid, s) : void()), ...);
}


hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.n_split < 1 || a.tile_lo < 0 || a.tile_lo >= a.n_tiles || a.split_base < 0 ||
      a.split_base + a.n_split > a.n_split_total || (a.n_split_total > 1 && (!a.part_o || !a.part_ml)))
    return hipErrorInvalidValue;
  if (a.psac_rank > 0) {
    TimedLaunch tl_("k_qu", s);
    const int64_t n = (int64_t)a.H * a.Nq;
    if (a.q.dtype == 0)
      hipLaunchKernelGGL(k_qu<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.q, a.H, a.Nq, a.psac_rank, a.U, a.qu,
                         a.range);
    else
      hipLaunchKernelGGL(k_qu<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.q, a.H, a.Nq, a.psac_rank, a.U, a.qu,
                         a.range);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int q_tiles = (a.Nq + kBM - 1) / kBM;
  const dim3 grid((unsigned)(q_tiles * a.n_split * a.H));
  const int flags = (a.q.dtype == 0 ? 1 : 0) | (a.k_mode == 1 ? 2 : 0) | (a.k_mode == 2 ? 32 : 0) |
                    (a.v_uniform_int2_1stage ? 4 : 0) |
                    (a.logits ? 8 : 0) | (a.psac_rank > 0 ? 16 : 0) | (a.kf.ptr ? 64 : 0);
  {
    TimedLaunch tl_("k_attend", s);
    if (flags & 64) {
      launch_attend_variant(flags, a, grid, s,
                            std::integer_sequence<int, 64, 68, 72, 76, 80, 84, 88, 92, 66, 70, 74, 78, 82, 86, 90, 94,
                                                  96, 100, 104, 108>{});
    } else if (flags & 32) {
      launch_attend_variant(flags, a, grid, s, std::integer_sequence<int, 32, 36, 40, 44>{});
    } else {
      launch_attend_variant(flags, a, grid, s, std::make_integer_sequence<int, 32>{});
    }
  }
  hipError_t e = hipGetLastError();
  // the merge follows the launch that writes the last partial rows
  if (e != hipSuccess || a.n_split_total == 1 || a.split_base + a.n_split < a.n_split_total) return e;
  const int64_t total = (int64_t)a.H * a.Nq * (kHeadDim / 4);
  TimedLaunch tl_("k_merge", s);
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qkv
