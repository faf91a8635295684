// k-means of one chunk's tokens per head: strided init, MFMA distance GEMM with
// wave argmin (assign), exact-sum centroid means (update).
//
// Method: Quant VideoGen notes, "Key designs / Semantic-Aware Smoothing" (the
// chunk's tokens are grouped by k-means and each group gets its mean as a
// centroid); QuantWM summary, "QuantWM", first technique (QSAC: per-channel
// query-activity weights w in the distance).
//
// Assign computes, for every token y and centroid c,
//     D'(y, c) = sum_k w_k c_k^2 + sum_k y_k (-2 w_k c_k)
// which differs from the weighted squared distance by sum_k w_k y_k^2, a
// per-token constant that does not move the argmin.  The dot products run on
// MFMA (v_mfma_f32_32x32x16_bf16), the accumulators starting from the norms:
// fp32(-2*w*c) is split into bf16 hi + lo (16
// significant bits), bf16 tokens are exact operands, fp32 tokens are split
// into hi + lo too (three products: hh, lh, hl); products are exact and the
// sums are fp32.  screen_threshold() bounds the screening error rigorously
// (the derivation is beside it); every token whose two best screened values
// are not farther apart than that bound is a close call.  At the end of the
// kernel a second screened sweep over the close calls lists the centroids
// within the bound of the best, and those are compared in the definition's
// own float64 arithmetic (channel order, each operation rounded once).  So
// the labels are those of the float64 definition, ties to the lowest index.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

__device__ __forceinline__ TensorView item_view(const KmBatch& b, const KmItem& it) {
  return TensorView{it.y, b.dtype, b.N, it.stride_token, it.stride_head};
}

constexpr int kPitch = 136;          // LDS row pitch (bf16): 128 + 8 keeps ds_read_b128 conflict-free

template <bool F32>
__device__ __forceinline__ float load1(const TensorView& y, int64_t tok, int h, int k) {
  const int64_t off = tok * y.stride_token + (int64_t)h * y.stride_head + k;
  if constexpr (F32) return reinterpret_cast<const float*>(y.ptr)[off];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(y.ptr)[off]);
}

// Block (head, 8 centroids): c_j = y[j * floor(N / C)] as float32.
template <bool F32>
__global__ __launch_bounds__(256) void k_init(KmBatch b) {
  const KmItem& it = b.it[blockIdx.z];
  const TensorView y = item_view(b, it);
  const int C = b.C;
  float* __restrict__ c = it.c;
  const int h = blockIdx.y;
  // the head's magnitude range starts empty (the incremental updates' record)
  if (blockIdx.x == 0 && it.emag) it.emag[(int64_t)h * 2 * kHeadDim + threadIdx.x] = 0u;   // 256 = 2 x 128 words
  if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0 && it.amb_count) *it.amb_count = 0;   // the first assign's count
  if (blockIdx.x == 0 && h == 0 && threadIdx.x < 2 && it.hlist) it.hlist[threadIdx.x] = 0u;   // k_cert's lists
  const int j = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (j >= C) return;
  const int64_t step = y.n_tokens / C;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = (threadIdx.x & 31) * 4 + e;
    c[((int64_t)h * C + j) * kHeadDim + k] = load1<F32>(y, (int64_t)j * step, h, k);
  }
}

// Screening bound of the assign.  For a token y and centroid c (weights
// w >= 0; ||.|| the w-weighted norm) the screened value is s = cn + the fp32
// MFMA sum of y times the bf16 pieces of fp32(-2 w c), cn = fp32(||c||^2).
// Its error against ||c||^2 - 2<y, c> is at most kT * 2||y|| ||c|| +
// kC * ||c||^2 (u = 2^-24; every fp32 addition inside the MFMAs taken as
// rounded within 2u, in any order, so n summed terms add (n-1) 2u / (1 -
// (n-1) 2u) of their magnitudes; Cauchy-Schwarz bounds sum |2 w y c| by
// 2||y|| ||c||):
//   bf16 tokens: the hi + lo pieces hold fp32(-2wc) to 2^-16, its rounding
//     adds u, and the 257 accumulated terms add 3.06e-5 of cn + 1.008 T:
//     kT = 4.7e-5, kC = 3.1e-5;
//   fp32 tokens: the token's own split and the dropped lo*lo product add
//     2 * 2^-16, and the 385 terms add 4.58e-5: kT = 9.3e-5, kC = 4.6e-5.
// Let b be the screened winner and D the exact distances.  e_b is bounded
// with c_b's own norm.  A centroid j with D_j <= D_b has ||c_j|| <= ||y|| +
// sqrt(D_b) (triangle inequality) and ||c_j|| <= the head's largest centroid
// norm; with r the smaller of the two, e_j <= kT 2||y|| r + kC r^2.  So s_j <=
// s_b + e_b + e_j <= s_b + thr, and when every other screened value exceeds
// s_b + thr, b is the unique minimiser of the exact distances -- and of the
// float64 ones of the definition, whose ~1e-14 relative rounding the 2^-40
// term covers.  D_b <= s_b + ||y||^2 + e_b; ||y||^2 (fp32 sums) carries a
// 2^-12 margin, cn and the largest norm 2^-20, the evaluation of thr 2^-10,
// and 2^-100 (1 + ||y||) covers products below fp32's normal range.
// scb = sqrtf(cn_b * (1 + 2^-20)) and rcm = sqrtf(cmax2 * (1 + 2^-20)) come
// precomputed (per centroid and per head).
template <bool F32>
__device__ __forceinline__ float screen_threshold(float yn, float s_b, float cn_b, float scb, float rcm) {
  constexpr float kT = F32 ? 9.3e-5f : 4.7e-5f, kC = F32 ? 4.6e-5f : 3.1e-5f;
  const float ynu = yn * (1.0f + 0x1p-12f), ry = sqrtf(ynu);
  const float cb = cn_b * (1.0f + 0x1p-20f);
  const float eb = 2.0f * kT * ry * scb + kC * cb;
  const float db = (fmaxf(s_b + ynu, 0.0f) + eb) * (1.0f + 0x1p-12f);
  const float r = fminf(ry + sqrtf(db), rcm);
  const float ej = 2.0f * kT * ry * r + kC * r * r;
  return (eb + ej) * (1.0f + 0x1p-10f) + 0x1p-40f * (ynu + db) + 0x1p-100f * (1.0f + ry);
}

// Assign: one workgroup per (head, range of 32-token sub-blocks), eight waves.
// The head's operand planes (2 x C rows of 128 bf16, ~136 KB padded) are
// formed in LDS from the centroids once and stay resident; each wave then sweeps all centroid
// blocks for 64 tokens at a time (fp32 tokens: 32).  bf16 sweeps are
// software-pipelined: the MFMAs of centroid block k + 1 alternate with the
// screening of block k, and the next item's tokens load into the operand
// registers once the last block's MFMAs are issued.  Close calls go to an LDS
// list and are re-decided at the end of the workgroup.
constexpr int kAsgWaves = 8;
constexpr int kAsgThreads = kAsgWaves * 64;
constexpr int kAsgMaxC = 256;
constexpr int kAsgList = 3072;        // LDS close-call list; beyond it a wave re-decides on the spot
constexpr int kCand = 16;             // candidates listed per close call; more: decided over all centroids
constexpr int kRsw = kAsgWaves * 32;  // close calls per round of the second sweep
constexpr int kAsgCUs = 256;
constexpr int kAsgUnitCost = 25;

template <bool F32>
__global__ __launch_bounds__(kAsgThreads) void k_assign(KmBatch b, int G) {
  const KmItem& it = b.it[blockIdx.y];
  const TensorView y = item_view(b, it);
  const int C = b.C, n_heads = b.H;
  const float* __restrict__ w = it.w;
  const float* __restrict__ cent = it.c;
  uint8_t* __restrict__ labels = it.labels;
  int* __restrict__ amb_count = it.amb_count;
  float* const ynbuf = it.ynorm;
  __shared__ __attribute__((aligned(16))) uint16_t sP[2][kAsgMaxC][kPitch];
  __shared__ __attribute__((aligned(16))) float sCn[kAsgMaxC];
  __shared__ float sCnS[kAsgMaxC];               // sqrtf(cn * (1 + 2^-20)), for the screening bound
  __shared__ __attribute__((aligned(16))) float sW[kHeadDim];
  __shared__ int sAmb[kAsgList];
  __shared__ int sAmbN, sNext;
  __shared__ uint8_t sCand[kRsw][kCand];
  __shared__ int sCandN[kRsw], sOvf[kRsw];
  __shared__ int sOvfN;
  const uint32_t logical = xcd_remap(blockIdx.x, (uint32_t)(G * n_heads));
  const int h = logical / G, g = logical % G;
  const int N = (int)y.n_tokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = (N + 31) >> 5;
  const int sb0 = (int)((int64_t)S * g / G), sb1 = (int)((int64_t)S * (g + 1) / G);
  // items: pairs of sub-blocks (fp32 tokens: single ones), an odd last one
  // alone; wave w starts with item w, then takes the next one from an LDS
  // counter, so the waves finish together
  constexpr int kPer = F32 ? 1 : 2;
  const int nsb = sb1 - sb0;
  const int npair = F32 ? 0 : nsb >> 1, nitems = F32 ? nsb : npair + (nsb & 1);
  const int Cp = (C + 31) & ~31;                 // whole 32-row blocks; rows past C never win (norm +inf)
  const int Cs = F32 ? Cp : (C + 63) & ~63;      // rows of the main sweep (bf16: an even block count)
  const uint16_t* y16 = reinterpret_cast<const uint16_t*>(y.ptr);
  const int64_t hoff = (int64_t)h * y.stride_head + half * 8;

  // bf16 tokens of one item: always two sub-blocks, rows clamped to the
  // head's last token (an odd last sub-block computes a spare one whose
  // results are dropped)
  uint4 raw[2][8];
  auto load_tokens = [&](int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t base = (int64_t)min(sb * 32 + t * 32 + col, N - 1) * y.stride_token + hoff;
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[t][s] = *reinterpret_cast<const uint4*>(y16 + base + s * 16);
    }
  };

  {
    // The head's operand planes and norms are formed here from the fp32
    // centroids: thread t takes half a row (centroid t / 2, channels
    // 64 (t % 2) .. + 63), writes bf16 hi and lo of fp32(-2 w c) into the LDS
    // planes and sums w c^2 in float64 with its partner lane, rounded to fp32
    // (the screening bound carries 2^-20 on the norms).  Rows in [C, Cs) have
    // zero planes and norm +inf, so they never win.  The weights arrive in
    // LDS by asynchronous copy for the rest of the kernel.  The first item's
    // tokens are requested first, so their latency overlaps the centroids'.
    if constexpr (!F32) load_tokens(sb0 + kPer * wave);      // past the range: clamped, unused
    if (wave == 1) {
      if (w) {
        dma4(w + h * kHeadDim + lane, &sW[0]);        // lane i lands at sW[i]
        dma4(w + h * kHeadDim + 64 + lane, &sW[64]);
      } else {
        sW[lane] = 1.0f;
        sW[64 + lane] = 1.0f;
      }
    } else if (wave == 2 && lane == 0) {
      sAmbN = 0;
      sNext = kAsgWaves;
    }
    {
      const int j = tid >> 1, k0 = (tid & 1) * 64;
      double nrm = 0.0;
      if (j < C) {
        const float4* cr = reinterpret_cast<const float4*>(cent + ((int64_t)h * C + j) * kHeadDim + k0);
        const float4* wr = w ? reinterpret_cast<const float4*>(w + h * kHeadDim + k0) : nullptr;
#pragma unroll
        for (int q = 0; q < 8; ++q) {                      // 8 channels per step
          const float4 ca = cr[2 * q], cb = cr[2 * q + 1];
          const float4 wa = wr ? wr[2 * q] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
          const float4 wb = wr ? wr[2 * q + 1] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
          const float cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
          const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
          u16x8 hi8, lo8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float bb = -2.0f * (wv[e] * cv[e]);      // exact doubling: the planes carry -2 w c
            const uint32_t hb = f32_to_bf16_bits(bb);
            hi8[e] = (uint16_t)hb;
            lo8[e] = (uint16_t)f32_to_bf16_bits(bb - bf16_bits_to_f32(hb));
            nrm += (double)wv[e] * ((double)cv[e] * (double)cv[e]);
          }
          *reinterpret_cast<u16x8*>(&sP[0][j][k0 + q * 8]) = hi8;
          *reinterpret_cast<u16x8*>(&sP[1][j][k0 + q * 8]) = lo8;
        }
      } else if (j < Cs) {
        const u16x8 z = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          *reinterpret_cast<u16x8*>(&sP[0][j][k0 + q * 8]) = z;
          *reinterpret_cast<u16x8*>(&sP[1][j][k0 + q * 8]) = z;
        }
      }
      nrm += __shfl_xor(nrm, 1);
      if ((tid & 1) == 0 && j < Cs) sCn[j] = j < C ? (float)nrm : INFINITY;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));               // the weights' copies
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // largest centroid norm of the head (wave-uniform; rows past C hold +inf)
  float cmax2 = 0.0f;
  for (int j = lane; j < C; j += 64) cmax2 = fmaxf(cmax2, sCn[j]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, o));
  cmax2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cmax2)));
  const float rcm = sqrtf(cmax2 * (1.0f + 0x1p-20f));
  if (tid < C) sCnS[tid] = sqrtf(sCn[tid] * (1.0f + 0x1p-20f));
  __syncthreads();

  // One wave decides token tok over all centroids, lanes over centroids, in
  // the definition's arithmetic: the sum over channels, in order, of
  // w_k (y_k - c_k)^2, each float64 operation rounded once; the lowest wins,
  // ties to the lowest index.  Called wave-uniformly.
  auto decide_all = [&](int tok) __attribute__((always_inline)) {
    const int64_t off = (int64_t)tok * y.stride_token + (int64_t)h * y.stride_head + lane * 2;
    float ya, yb;
    if constexpr (F32) {
      const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(y.ptr) + off);
      ya = v.x;
      yb = v.y;
    } else {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(y16 + off);
      ya = bf16_bits_to_f32(v & 0xFFFFu);
      yb = bf16_bits_to_f32(v >> 16);
    }
    double best = INFINITY;
    int bj = 0;
    for (int q = 0; q < kAsgMaxC / 64; ++q) {
      const int j = q * 64 + lane;
      const float* cr = cent + ((int64_t)h * C + min(j, C - 1)) * kHeadDim;
      double dist = 0.0;
#pragma unroll 8
      for (int k = 0; k < kHeadDim; k += 2) {
        const float yk0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ya), k >> 1));
        const float yk1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, yb), k >> 1));
        const float2 cv = *reinterpret_cast<const float2*>(cr + k);
        const double d0 = (double)yk0 - (double)cv.x, d1 = (double)yk1 - (double)cv.y;
        dist += (double)sW[k] * (d0 * d0);
        dist += (double)sW[k + 1] * (d1 * d1);
      }
      if (j < C && dist < best) {
        best = dist;
        bj = j;
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double ov = __shfl_xor(best, o);
      const int oj = __shfl_xor(bj, o);
      if (ov < best || (ov == best && oj < bj)) {
        best = ov;
        bj = oj;
      }
    }
    if (lane == 0) labels[(int64_t)h * N + tok] = (uint8_t)bj;
  };

  for (int it = wave; it < nitems;) {
    const int sb = sb0 + kPer * it, nt = it < npair ? 2 : 1;
    const int tok0 = sb * 32;
    int next = 0;
    if (lane == 0) next = atomicAdd(&sNext, 1);
    next = __builtin_amdgcn_readfirstlane(next);
    // B operand (tokens): lane holds token tok0 + t*32 + col, channels s*16 + half*8 + [0, 8).
    // ynorm[t] = sum_k w_k y_k^2 over the lane's channels (fp32; it only sets
    // the screening threshold).
    bf16x8 yh[2][8];
    bf16x8 yl[2][F32 ? 8 : 1];
    float ynorm[2] = {0.0f, 0.0f};
    // bf16 tokens after the first iteration: ||y||^2 from the first (it does
    // not change within a stage)
    const bool cached = !F32 && b.iter > 0 && ynbuf != nullptr;
    float ync[2] = {0.0f, 0.0f};
    if constexpr (F32) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        const int tok = tok0 + t * 32 + col;
        const bool ok = tok < N;
        const float* p = reinterpret_cast<const float*>(y.ptr) + (int64_t)min(tok, N - 1) * y.stride_token + hoff;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int ch = s * 16 + half * 8;
          float4 a = *reinterpret_cast<const float4*>(p + s * 16);
          float4 b = *reinterpret_cast<const float4*>(p + s * 16 + 4);
          if (!ok) a = b = make_float4(0, 0, 0, 0);
          const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          u16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hb = f32_to_bf16_bits(v[e]);
            hi[e] = (uint16_t)hb;
            lo[e] = (uint16_t)f32_to_bf16_bits(v[e] - bf16_bits_to_f32(hb));
            ynorm[t] += sW[ch + e] * (v[e] * v[e]);
          }
          yh[t][s] = __builtin_bit_cast(bf16x8, hi);
          yl[t][F32 ? s : 0] = __builtin_bit_cast(bf16x8, lo);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s) yh[t][s] = as_bf16x8(raw[t][s]);
      if (cached) {
#pragma unroll
        for (int t = 0; t < 2; ++t) ync[t] = ynbuf[(int64_t)h * N + min(tok0 + t * 32 + col, N - 1)];
      } else if (w == nullptr) {                 // sum of squares by packed bf16 dot products
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const uint32_t r4[4] = {raw[t][s].x, raw[t][s].y, raw[t][s].z, raw[t][s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bf16x2 q = __builtin_bit_cast(bf16x2, r4[e]);
              part[e] = __builtin_amdgcn_fdot2_f32_bf16(q, q, part[e], false);
            }
          }
          ynorm[t] = (part[0] + part[1]) + (part[2] + part[3]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const uint32_t r4[4] = {raw[t][s].x, raw[t][s].y, raw[t][s].z, raw[t][s].w};
            const int ch = s * 16 + half * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = bf16_bits_to_f32((r4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
              ynorm[t] += sW[ch + e] * (v * v);
            }
          }
      }
    }

    int spill = 0;                               // 1 + token of a close call past the list
    // Sweep of the centroid blocks for NT sub-blocks: running best b1 and
    // second best b2 of the screened values (b1 <= b2; new b2 = med3(b1, b2, v),
    // new b1 = min(b1, v)).  rel is the best row relative
    // to the current block's first row, so each element selects a small
    // immediate; the lane's row offset half*4 is added at the end.
    auto sweep = [&](auto nt) __attribute__((always_inline)) {
      constexpr int NT = decltype(nt)::value;
      float b1[NT], b2[NT];
      int rel[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        b1[t] = INFINITY;
        b2[t] = INFINITY;
        rel[t] = 32;
      }
      // MFMAs of block cb; the accumulators start from ||c_j||_w^2 of their
      // centroid rows: row (r/4)*8 + half*4 + r%4 of the block for element r
      auto mma = [&](f32x16 (&acc)[NT], int cb) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 c4 = *reinterpret_cast<const float4*>(&sCn[cb + q * 8 + half * 4]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[t][4 * q] = c4.x;
            acc[t][4 * q + 1] = c4.y;
            acc[t][4 * q + 2] = c4.z;
            acc[t][4 * q + 3] = c4.w;
          }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const uint4*>(&sP[0][cb + col][s * 16 + half * 8]));
          const bf16x8 alo = as_bf16x8(*reinterpret_cast<const uint4*>(&sP[1][cb + col][s * 16 + half * 8]));
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yh[t][s], acc[t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, yh[t][s], acc[t], 0, 0, 0);
          if constexpr (F32) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yl[t][F32 ? s : 0], acc[t], 0, 0, 0);
          }
        }
      };
      // The same MFMAs for bf16 tokens, with explicit LDS bases (each plane
      // and the norms lie beyond the 16-bit offset field of one another, so
      // each gets its own base) and the next k-slice's operands requested one
      // slice ahead.
      auto mma_p = [&](f32x16 (&acc)[NT], int cb) __attribute__((always_inline)) {
        const uint4* ph = reinterpret_cast<const uint4*>(&sP[0][cb + col][half * 8]);
        const uint4* pl = reinterpret_cast<const uint4*>(&sP[1][cb + col][half * 8]);
        const float4* pn = reinterpret_cast<const float4*>(&sCn[cb + half * 4]);
        uint4 ah = ph[0], al = pl[0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 c4 = pn[2 * q];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[t][4 * q] = c4.x;
            acc[t][4 * q + 1] = c4.y;
            acc[t][4 * q + 2] = c4.z;
            acc[t][4 * q + 3] = c4.w;
          }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          uint4 nh = ah, nl = al;
          if (s + 1 < 8) {
            nh = ph[2 * (s + 1)];
            nl = pl[2 * (s + 1)];
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), yh[t][s], acc[t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), yh[t][s], acc[t], 0, 0, 0);
          ah = nh;
          al = nl;
        }
      };
      // rows increase with r within the lane, so strict '<' keeps the lowest
      // index among equal values
      auto top2 = [&](const f32x16 (&acc)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t) rel[t] -= 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = (r >> 2) * 8 + (r & 3);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float v = acc[t][r];
            const bool l = v < b1[t];
            b2[t] = __builtin_amdgcn_fmed3f(b1[t], b2[t], v);
            b1[t] = l ? v : b1[t];               // a select: min() would first quiet v
            rel[t] = l ? j : rel[t];
          }
        }
      };
      // One screening step of top2: value v (token sub-block v % NT, element v / NT).
      auto step = [&](const f32x16 (&acc)[NT], int v) __attribute__((always_inline)) {
        const int t = v % NT, r = v / NT;
        const int j = (r >> 2) * 8 + (r & 3);
        const float x = acc[t][r];
        const bool l = x < b1[t];
        b2[t] = __builtin_amdgcn_fmed3f(b1[t], b2[t], x);
        b1[t] = l ? x : b1[t];
        rel[t] = l ? j : rel[t];
      };
      // The MFMAs of block cbn into an (from the norms), each followed by one
      // screening step of ap, the previous block (same order of values as
      // top2, so the same result); the scheduling barriers keep that order,
      // so the matrix core runs while the wave screens.
      auto stage = [&](f32x16 (&an)[NT], int cbn, const f32x16 (&ap)[NT]) __attribute__((always_inline)) {
        const uint4* ph = reinterpret_cast<const uint4*>(&sP[0][cbn + col][half * 8]);
        const uint4* pl = reinterpret_cast<const uint4*>(&sP[1][cbn + col][half * 8]);
        const float4* pn = reinterpret_cast<const float4*>(&sCn[cbn + half * 4]);
        uint4 ah = ph[0], al = pl[0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 c4 = pn[2 * q];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            an[t][4 * q] = c4.x;
            an[t][4 * q + 1] = c4.y;
            an[t][4 * q + 2] = c4.z;
            an[t][4 * q + 3] = c4.w;
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) rel[t] -= 32;
#pragma unroll
        for (int v = 0; v < NT; ++v) step(ap, v);      // while the operands arrive
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          uint4 nh = ah, nl = al;
          if (s + 1 < 8) {
            nh = ph[2 * (s + 1)];
            nl = pl[2 * (s + 1)];
          }
#pragma unroll
          for (int pln = 0; pln < 2; ++pln) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              an[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pln ? al : ah), yh[t][s], an[t], 0, 0, 0);
              const int v = NT + (s * 2 + pln) * NT + t;
              if (v < 16 * NT) step(ap, v);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          ah = nh;
          al = nl;
        }
      };
      if constexpr (F32) {
        for (int cb = 0; cb < Cp; cb += 32) {
          f32x16 acc[NT];
          mma(acc, cb);
          top2(acc);
        }
      } else {
        // Software pipeline over the centroid blocks (stage): the MFMAs of
        // block k + 1 alternate with the screening of block k, so the matrix
        // core works while the wave screens.  After the last block's MFMAs
        // the token registers are free: the next item's tokens load into
        // them while the last block is screened.
        // The block count is even (Cs = Cp rounded up to 64 rows; the extra
        // rows hold copies of a valid row with norm +inf, so they never win
        // and leave the second best alone).
        f32x16 accA[NT], accB[NT];
        const int nb = Cs >> 5;
        mma_p(accA, 0);
        for (int k = 0; k + 2 < nb; k += 2) {    // blocks k (in accA), k + 1, k + 2
          stage(accB, (k + 1) * 32, accA);
          stage(accA, (k + 2) * 32, accB);
        }
        stage(accB, (nb - 1) * 32, accA);
        // the token registers are dead once the last block's MFMAs are issued
        // (unconditional, so no branch splits the stage from the screening:
        // past the last item a valid item is read again and not used)
        load_tokens(sb0 + kPer * min(next, nitems - 1));
        top2(accB);
      }
      int bidx[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bidx[t] = rel[t] + Cs - 32 + half * 4;
      // Close calls -- the two best screened values within the screening
      // error bound (screen_threshold) -- are listed for the float64
      // re-decision at the end.
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float o1 = __shfl_xor(b1[t], 32), o2 = __shfl_xor(b2[t], 32);
        const int oi = __shfl_xor(bidx[t], 32);
        const float second = fminf(fmaxf(b1[t], o1), fminf(b2[t], o2));
        if (o1 < b1[t] || (o1 == b1[t] && oi < bidx[t])) {
          b1[t] = o1;
          bidx[t] = oi;
        }
        const float yn = cached ? ync[t] : ynorm[t] + __shfl_xor(ynorm[t], 32);
        const int tok = tok0 + t * 32 + col;
        if (half == 0 && t < nt && tok < N) {
          labels[(int64_t)h * N + tok] = (uint8_t)bidx[t];
          if (!F32 && b.iter == 0 && ynbuf) ynbuf[(int64_t)h * N + tok] = yn;
          if (!(second - b1[t] > screen_threshold<F32>(yn, b1[t], sCn[bidx[t]], sCnS[bidx[t]], rcm))) {
            const int slot = atomicAdd(&sAmbN, 1);
            if (slot < kAsgList) sAmb[slot] = tok;
            else spill = tok + 1;
          }
        }
      }
    };
    if constexpr (F32) sweep(std::integral_constant<int, 1>{});
    else sweep(std::integral_constant<int, 2>{});
    // the list is full (a pathological input): this wave decides its
    // overflowing close calls one at a time over all centroids
    for (uint64_t m = __ballot(spill != 0); m; m &= m - 1) {
      const int src = __builtin_ctzll(m);
      decide_all(__builtin_amdgcn_readlane(spill, src) - 1);
    }
    it = next;
  }

  // Close calls.  A second screened sweep over them (32 per wave, the same
  // MFMAs) lists every centroid j with s_j - s_b <= thr: by the bound of
  // screen_threshold these include every centroid whose exact distance is not
  // above the winner's, so the float64 minimiser of the definition is among
  // them.  The candidates are evaluated in the definition's arithmetic (the
  // sum over channels, in order, of w_k (y_k - c_k)^2, each float64 operation
  // rounded once) and the lowest wins, ties to the lowest index.  A token with
  // more than kCand candidates is decided over all centroids by one wave.
  __syncthreads();
  const int n_amb = min(sAmbN, kAsgList);
  if (n_amb > 0 && tid == 0 && amb_count) atomicAdd(amb_count, n_amb);   // statistics only
  for (int e0 = 0; e0 < n_amb; e0 += kRsw) {
    const int nloc = min(kRsw, n_amb - e0);
    if (tid < kRsw) sCandN[tid] = 0;
    if (tid == 0) sOvfN = 0;
    __syncthreads();
    if (wave * 32 < nloc) {                                  // wave-uniform
      const int loc = wave * 32 + col;
      const bool live = loc < nloc;
      const int tok = sAmb[e0 + min(loc, nloc - 1)];
      const int64_t base = (int64_t)tok * y.stride_token + hoff;
      bf16x8 rh[8], rl[F32 ? 8 : 1];
      float yn = 0.0f;                                       // sum_k w_k y_k^2 (fp32; sets the bound only)
      if constexpr (F32) {
        const float* p = reinterpret_cast<const float*>(y.ptr) + base;
#pragma unroll
        for (int sI = 0; sI < 8; ++sI) {
          const float4 a = *reinterpret_cast<const float4*>(p + sI * 16);
          const float4 b = *reinterpret_cast<const float4*>(p + sI * 16 + 4);
          const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          u16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hb = f32_to_bf16_bits(v[e]);
            hi[e] = (uint16_t)hb;
            lo[e] = (uint16_t)f32_to_bf16_bits(v[e] - bf16_bits_to_f32(hb));
            yn += sW[sI * 16 + half * 8 + e] * (v[e] * v[e]);
          }
          rh[sI] = __builtin_bit_cast(bf16x8, hi);
          rl[sI] = __builtin_bit_cast(bf16x8, lo);
        }
      } else {
#pragma unroll
        for (int sI = 0; sI < 8; ++sI) {
          const uint4 raw4 = *reinterpret_cast<const uint4*>(y16 + base + sI * 16);
          rh[sI] = as_bf16x8(raw4);
          const uint32_t r4[4] = {raw4.x, raw4.y, raw4.z, raw4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = bf16_bits_to_f32((r4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            yn += sW[sI * 16 + half * 8 + e] * (v * v);
          }
        }
      }
      yn += __shfl_xor(yn, 32);
      // screened values of block cb (the same MFMAs as the sweep)
      auto block = [&](int cb) __attribute__((always_inline)) -> f32x16 {
        f32x16 acc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 c4 = *reinterpret_cast<const float4*>(&sCn[cb + q * 8 + half * 4]);
          acc[4 * q] = c4.x;
          acc[4 * q + 1] = c4.y;
          acc[4 * q + 2] = c4.z;
          acc[4 * q + 3] = c4.w;
        }
#pragma unroll
        for (int sI = 0; sI < 8; ++sI) {
          const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const uint4*>(&sP[0][cb + col][sI * 16 + half * 8]));
          const bf16x8 alo = as_bf16x8(*reinterpret_cast<const uint4*>(&sP[1][cb + col][sI * 16 + half * 8]));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rh[sI], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, rh[sI], acc, 0, 0, 0);
          if constexpr (F32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rl[F32 ? sI : 0], acc, 0, 0, 0);
        }
        return acc;
      };
      // pass 1: the screened winner (value, lowest index) and its bound
      float m1 = INFINITY;
      int b1j = 0;
      for (int cb = 0; cb < Cp; cb += 32) {
        const f32x16 acc = block(cb);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = cb + (r >> 2) * 8 + half * 4 + (r & 3);
          if (acc[r] < m1) {                                 // rows rise with r and cb: ties keep the lowest
            m1 = acc[r];
            b1j = j;
          }
        }
      }
      {
        const float om = __shfl_xor(m1, 32);
        const int oj = __shfl_xor(b1j, 32);
        if (om < m1 || (om == m1 && oj < b1j)) {
          m1 = om;
          b1j = oj;
        }
      }
      const float thr = screen_threshold<F32>(yn, m1, sCn[min(b1j, C - 1)], sCnS[min(b1j, C - 1)], rcm);
      // pass 2: every centroid within the bound of the winner
      for (int cb = 0; cb < Cp; cb += 32) {
        const f32x16 acc = block(cb);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = cb + (r >> 2) * 8 + half * 4 + (r & 3);
          if (live && j < C && acc[r] - m1 <= thr) {
            const int n = atomicAdd(&sCandN[loc], 1);
            if (n < kCand) sCand[loc][n] = (uint8_t)j;
          }
        }
      }
    }
    __syncthreads();
    {
      // thread pair (loc, sub) evaluates candidates sub, sub + 2, ... of close call loc
      const int loc = tid >> 1, sub = tid & 1;
      if (loc < nloc) {
        const int cnt = sCandN[loc];
        const int tok = sAmb[e0 + loc];
        if (cnt > kCand || cnt == 0) {                       // none: a NaN bound
          if (sub == 0) sOvf[atomicAdd(&sOvfN, 1)] = tok;
        } else {
          constexpr int kMine = kCand / 2;
          const int my = (cnt - sub + 1) >> 1;
          double dist[kMine];
          int jj[kMine];
#pragma unroll
          for (int n = 0; n < kMine; ++n) {
            dist[n] = 0.0;
            jj[n] = n < my ? (int)sCand[loc][sub + 2 * n] : 0;
          }
          const int64_t base = (int64_t)tok * y.stride_token + (int64_t)h * y.stride_head;
#pragma unroll 1
          for (int g = 0; g < kHeadDim / 16; ++g) {
            float yv[16];
            if constexpr (F32) {
              const float* p = reinterpret_cast<const float*>(y.ptr) + base + g * 16;
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const float4 v = *reinterpret_cast<const float4*>(p + 4 * x);
                yv[4 * x] = v.x;
                yv[4 * x + 1] = v.y;
                yv[4 * x + 2] = v.z;
                yv[4 * x + 3] = v.w;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) yv[e] = bf16_bits_to_f32(y16[base + g * 16 + e]);
            }
#pragma unroll
            for (int n = 0; n < kMine; ++n) {
              if (n < my) {
                const float* cr = cent + ((int64_t)h * C + jj[n]) * kHeadDim + g * 16;
                float cv[16];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                  const float4 v = *reinterpret_cast<const float4*>(cr + 4 * x);
                  cv[4 * x] = v.x;
                  cv[4 * x + 1] = v.y;
                  cv[4 * x + 2] = v.z;
                  cv[4 * x + 3] = v.w;
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                  const double df = (double)yv[e] - (double)cv[e];
                  const double sq = df * df;
                  dist[n] = dist[n] + (double)sW[g * 16 + e] * sq;
                }
              }
            }
          }
          double best = INFINITY;
          int bj = 0x7fffffff;
#pragma unroll
          for (int n = 0; n < kMine; ++n)
            if (n < my && (dist[n] < best || (dist[n] == best && jj[n] < bj))) {
              best = dist[n];
              bj = jj[n];
            }
          const double ob = __shfl_xor(best, 1);
          const int oj = __shfl_xor(bj, 1);
          if (ob < best || (ob == best && oj < bj)) {
            best = ob;
            bj = oj;
          }
          if (sub == 0) labels[(int64_t)h * N + tok] = (uint8_t)bj;
        }
      }
    }
    __syncthreads();
    for (int o = wave; o < sOvfN; o += kAsgWaves) decide_all(sOvf[o]);   // block-uniform bound
    __syncthreads();
  }
}

// The head-wide certificate of the incremental update, per channel over all
// of the head's tokens (emag, recorded by the first update of the stage):
// every nonzero bf16 magnitude is an integer multiple of 2^(emin - 134) and
// below 2^(emax - 126) (biased exponents of the smallest nonzero and the
// largest magnitude), so a signed sum of at most N of them is an integer
// multiple of that unit below 2^(emax - emin + lg + 8) units, lg >= log2 N:
// exact in float64 when emax - emin + lg <= 44 (the bound of the per-cluster
// certificate, with N for the cluster size).  Every intermediate value of an
// incremental update is such a sum (a set of distinct tokens), so the sums it
// keeps are the exact sums.  Wave-uniform.
__device__ __forceinline__ bool head_span_ok(const KmItem& it, int h, int N, int limit) {
  const int lane = threadIdx.x & 63;
  const int lg = 32 - __builtin_clz((unsigned)max(N, 1));
  bool ok = true;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int k = q * 64 + lane;
    const uint32_t mx = it.emag[(int64_t)h * 2 * kHeadDim + k];
    const uint32_t mn = 0xFFFFu - it.emag[((int64_t)h * 2 + 1) * kHeadDim + k];   // min nonzero magnitude - 1
    const int emax = (int)(mx >> 7), emin = max((int)(((mn + 1u) >> 7) & 0xFFu), 1);
    ok = ok && (mn == 0xFFFFu || (emax < 0xFF && emax - emin + lg <= limit));
  }
  return __ballot(!ok) == 0;
}

// The head's classes: 1 when float64 sums are exact (the bound 44 above); 2
// when 64-bit integer sums in units of 2^(emin - 134) are: a signed sum of at
// most N values is then below 2^(emax - emin + 8 + lg) units, within int64
// when emax - emin + lg <= 55; 0 otherwise (the full update every iteration).
constexpr uint32_t kCertF64 = 1, kCertFix = 2;

// Smallest nonzero biased exponent of channel k of head h (1 for subnormals
// and for an all-zero channel), from the recorded range.
__device__ __forceinline__ int chan_emin(const KmItem& it, int h, int k) {
  const uint32_t mn = 0xFFFFu - it.emag[((int64_t)h * 2 + 1) * kHeadDim + k];
  return max((int)(((mn + 1u) >> 7) & 0xFFu), 1);
}
// bf16 bits b as a signed integer number of units 2^(emin - 134) (exact: the
// value's exponent is at least emin).
__device__ __forceinline__ int64_t fix_of(uint32_t b, int emin) {
  const uint32_t E = (b >> 7) & 0xFFu, f = b & 0x7Fu;
  const int64_t m = (int64_t)(E ? (f | 0x80u) : f);
  const int sh = max((E ? (int)E : 1) - emin, 0);
  return (b & 0x8000u) ? -(m << sh) : (m << sh);
}
// The float64 rounding of the integer sum s units of 2^(emin - 134): both
// 32-bit halves convert exactly, their sum rounds once, the scaling is exact.
__device__ __forceinline__ double fix_to_f64(int64_t s, int emin) {
  const double hi = (double)(int32_t)(s >> 32) * 4294967296.0, lo = (double)(uint32_t)(s & 0xFFFFFFFFll);
  return ldexp(hi + lo, emin - 134);
}
// Whether the grouping and the full update take head h in iteration b.iter
// of an incremental stage (inc == 2): the heads outside both classes always;
// the fixed-point class in its first later iteration, which also records its
// integer sums; never the float64 class.
__device__ __forceinline__ bool full_update_takes(const KmBatch& b, uint32_t cert) {
  return cert == 0 || (cert == kCertFix && b.iter == 1);
}

// Centroid j of head h from its exact sum (channels c4 .. c4 + 3 per lane):
// c = fl32(sum / n).  (The assign forms its operand planes and norms from c.)
__device__ __forceinline__ void centroid_from_sum(const KmItem& it, int h, int C, int j, int c4, const double* sv,
                                                  int n) {
  float cv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cv[e] = (float)(sv[e] / (double)n);
  *reinterpret_cast<float4*>(it.c + ((int64_t)h * C + j) * kHeadDim + c4) = make_float4(cv[0], cv[1], cv[2], cv[3]);
}

// Centroid update fused with the grouping of tokens by label.  One workgroup
// per (head, 8 consecutive clusters); wave w owns clusters 2w and 2w + 1 of
// the group.  The head's labels are scanned in windows of kUpdWindow tokens:
// the members of the group's clusters in the window are listed in LDS
// (counting sort), then each wave adds its clusters' member rows (each lane
// two channels).  The sums must be exact (their float64 rounding is then the
// correctly rounded sum whatever the order; the mean is rounded once more to
// float32):
//  - bf16 tokens in one window: plain float64 sums, with a certificate: every
//    partial sum of n values of 8-bit significands is an integer multiple of
//    the smallest significand unit, below n * 2^(emax+1), so it is exact when
//    emax - emin + ceil(log2 n) <= 44 (biased exponents of the largest and the
//    smallest nonzero magnitude, tracked with packed 16-bit min/max); a
//    channel that fails it is summed again in double-double;
//  - otherwise double-double throughout (exact up to ~2^-104 relative).
// An empty cluster keeps its centroid.
constexpr int kUpdClusters = 8;
constexpr int kUpdClustersG = 32;       // clusters per workgroup when the member lists come from k_group
constexpr int kUpdWindow = 8192;          // token index << 3 fits 16 bits
static_assert(kUpdWindow == kGroupMaxTokens, "grouped heads fit one update window");
constexpr int kUpdRows = 12;            // member-row loads in flight per lane group
constexpr int kListGroupGrid = 256;     // workgroups of the list-driven grouping and update
constexpr int kListUpdateGrid = 1024;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Grouping of a head's tokens by label for the update (counting sort): one
// workgroup per (problem, head of at most kUpdWindow tokens) writes the cluster
// offsets [C + 1] and the token list ordered by cluster, so that the update's
// workgroups (32 per head) read their clusters' members instead of each
// scanning all labels.
__device__ __forceinline__ void group_head(const KmBatch& b, int pi, int h) {
  const KmItem& it = b.it[pi];
  const int C = b.C, N = (int)b.N;
  __shared__ int s_c[256], s_o[257];
  __shared__ uint16_t s_l[kUpdWindow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t cert = b.inc == 2 ? it.cert[h] : 0u;
  if (b.inc == 2 && !full_update_takes(b, cert)) return;   // the incremental update takes this head
  const uint8_t* lab = it.labels + (int64_t)h * N;
  // before a head's first incremental update (the stage's first update, or a
  // fixed-point head's first full one after it) these labels are the previous
  // ones of the next update (alternate buffer (iter + 1) & 1)
  uint8_t* rec = b.inc == 1 || (b.inc == 2 && cert == kCertFix)
                     ? it.prev + ((int64_t)((b.iter + 1) & 1) * b.H + h) * N : nullptr;
  uint32_t kk[kUpdWindow / 256];                 // labels of tokens tid*32 .. tid*32 + 31
  {
    const int i0 = tid * 32;
    if ((N & 3) == 0 && i0 + 32 <= N) {
      uint32_t wv[8];
      const uint32_t* l4 = reinterpret_cast<const uint32_t*>(lab + i0);
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[q] = l4[q];
      if (rec) {
#pragma unroll
        for (int q = 0; q < 8; ++q) reinterpret_cast<uint32_t*>(rec + i0)[q] = wv[q];
      }
#pragma unroll
      for (int x = 0; x < 32; ++x) kk[x] = (wv[x >> 2] >> (8 * (x & 3))) & 0xFFu;
    } else {
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        const int i = i0 + x;
        const uint32_t l = lab[min(i, N - 1)];
        kk[x] = i < N ? l : 0xFFFFFFFFu;
        if (rec && i < N) rec[i] = (uint8_t)l;
      }
    }
  }
  s_c[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 32; ++x)
    if (kk[x] < (uint32_t)C) atomicAdd(&s_c[kk[x]], 1);
  __syncthreads();
  if (wave == 0) {                               // exclusive prefix over the clusters, four per lane
    int a[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = s_c[lane * 4 + e];
      sum += a[e];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int ex = incl - sum;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_o[lane * 4 + e] = ex;
      s_c[lane * 4 + e] = ex;                    // the cursor of the scatter
      ex += a[e];
    }
    if (lane == 63) s_o[256] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 32; ++x)
    if (kk[x] < (uint32_t)C) s_l[atomicAdd(&s_c[kk[x]], 1)] = (uint16_t)(tid * 32 + x);
  __syncthreads();
  for (int k = tid; k <= C; k += 256) it.grp_off[(int64_t)h * (C + 1) + k] = k < C ? s_o[k] : s_o[256];
  for (int e = tid; e < N; e += 256) it.grp_list[(int64_t)h * N + e] = s_l[e];
}

__global__ __launch_bounds__(256) void k_group(KmBatch b) { group_head(b, blockIdx.y, blockIdx.x); }

// The heads that a later iteration's full update takes (inc == 2), from the
// per-problem lists that k_cert writes: those outside both certificate
// classes, and in iteration 1 the fixed-point heads as well.  The list
// kernels' workgroups stride over these heads (or (head, cluster group)
// items), problem after problem, so that iterations where no head needs the
// full update (the usual case) dispatch a few hundred workgroups, not one per
// head and cluster group.
__device__ __forceinline__ int listed_heads(const KmBatch& b, const KmItem& it) {
  return (int)min(it.hlist[0], (uint32_t)b.H) + (b.iter == 1 ? (int)min(it.hlist[1], (uint32_t)b.H) : 0);
}
__device__ __forceinline__ int listed_head(const KmBatch& b, const KmItem& it, int e) {
  const int n0 = (int)min(it.hlist[0], (uint32_t)b.H);
  return (int)(e < n0 ? it.hlist[2 + e] : it.hlist[2 + b.H + (e - n0)]);
}

// Every problem's item count (listed heads x per_head) into s_n, fetched at once.
__device__ __forceinline__ void listed_counts(const KmBatch& b, int per_head, int* s_n) {
  if (threadIdx.x < b.n) s_n[threadIdx.x] = listed_heads(b, b.it[threadIdx.x]) * per_head;
  __syncthreads();
}

__global__ __launch_bounds__(256) void k_group_list(KmBatch b) {
  __shared__ int s_n[kKmMaxBatch];
  listed_counts(b, 1, s_n);
  int e = blockIdx.x;
  for (int p = 0; p < b.n; ++p) {
    const KmItem& it = b.it[p];
    const int cnt = s_n[p];
    for (; e < cnt; e += gridDim.x) {
      group_head(b, p, listed_head(b, it, e));
      __syncthreads();                           // the LDS lists are rebuilt for the next head
    }
    e -= cnt;
  }
}

// clusters c0 .. c0 + CPG - 1 of head h of problem pi
template <bool F32, bool GROUPED, int CPG>
__device__ __forceinline__ void update_block(const KmBatch& b, int pi, int h, int c0) {
  const KmItem& it = b.it[pi];
  const TensorView y = item_view(b, it);
  const int C = b.C;
  const uint8_t* __restrict__ labels = it.labels;
  float* __restrict__ c = it.c;
  const float* __restrict__ w = it.w;
  int32_t* __restrict__ counts = it.counts;
  // CPG clusters per workgroup: with k_group's member lists one prologue
  // (offsets, then the list) can serve up to 32 clusters, which the waves take
  // two at a time in CPG / 8 sub-rounds; the label-scanning variant keeps 8
  // (3-bit cluster codes)
  static_assert(CPG % kUpdClusters == 0 && CPG <= kUpdClustersG && (GROUPED || CPG == kUpdClusters), "CPG");
  __shared__ int s_cnt[kUpdClusters], s_off[kUpdClustersG + 1], s_cur[kUpdClusters];
  __shared__ uint16_t s_mem[kUpdWindow];
  __shared__ int s_wtot[4];
  __shared__ uint32_t s_emag[2][kHeadDim];      // inc == 1: this workgroup's magnitude range per channel
  const int N = (int)y.n_tokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t cert = b.inc == 2 ? it.cert[h] : 0u;
  if (b.inc == 2 && !full_update_takes(b, cert)) return;   // the incremental update takes this head
  const bool record = GROUPED && !F32 && b.inc == 1;  // the first update of an incremental stage
  const bool record_fix = GROUPED && !F32 && b.inc == 2 && cert == kCertFix;   // integer sums, once
  if (record) s_emag[tid >> 7][tid & (kHeadDim - 1)] = 0u;   // 256 threads: both halves (synchronised below)
  const uint8_t* lab = labels + (int64_t)h * N;
  const int64_t hoff = (int64_t)h * y.stride_head + lane * 2;
  const bool plain = !F32 && N <= kUpdWindow;   // certified float64 sums
  DD acc[2][2] = {{{0.0, 0.0}, {0.0, 0.0}}, {{0.0, 0.0}, {0.0, 0.0}}};
  int total[2] = {0, 0};
  bool old_fin[2] = {true, true};               // finished after the window loop (2 channels per lane)

  // member rows [m0, m1) of the window list: value pairs (channels lane*2, +1)
  auto row_pair = [&](int t0, int mm, float& x0, float& x1) __attribute__((always_inline)) -> uint32_t {
    const int64_t off = (int64_t)(t0 + s_mem[mm]) * y.stride_token + hoff;
    if constexpr (F32) {
      const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(y.ptr) + off);
      x0 = v.x;
      x1 = v.y;
      return 0u;
    } else {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(y.ptr) + off);
      x0 = bf16_bits_to_f32(v & 0xFFFFu);
      x1 = bf16_bits_to_f32(v >> 16);
      return v;
    }
  };
  auto dd_rows = [&](int t0, int m0, int m1, DD& a0, DD& a1) __attribute__((always_inline)) {
    for (int m = m0; m < m1; m += 16) {
      float vx[16], vy[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) row_pair(t0, min(m + q, m1 - 1), vx[q], vy[q]);   // past the end: loaded, not added
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (m + q < m1) {
          a0.add((double)vx[q]);
          a1.add((double)vy[q]);
        }
      }
    }
  };

  // centroids of pair p (clusters c0 + 2p, + 1) summed in double-double: the
  // clusters the certificate did not cover, or every cluster of fp32 data
  auto finish_pair = [&](int p) __attribute__((always_inline)) {
    for (int cc = 0; cc < 2; ++cc) {
      const int j = c0 + p * 2 + cc;
      if (j >= C) continue;
      const int n = total[cc];
      if (counts && lane == 0) counts[h * C + j] = n;
      if (n == 0 || !old_fin[cc]) continue;
      const float cv[2] = {(float)(acc[cc][0].hi / (double)n), (float)(acc[cc][1].hi / (double)n)};
      *reinterpret_cast<float2*>(c + ((int64_t)h * C + j) * kHeadDim + lane * 2) = make_float2(cv[0], cv[1]);
    }
  };

  for (int t0 = 0; t0 < N; t0 += kUpdWindow) {
    if constexpr (GROUPED) {                     // the head's tokens already ordered by cluster (k_group)
      const int* go = it.grp_off + (int64_t)h * (C + 1);
      const int base = go[c0];
      const int M = go[min(c0 + CPG, C)] - base;
      if (tid <= CPG) s_off[tid] = go[min(c0 + tid, C)] - base;
      for (int e = tid; e < M; e += 256) s_mem[e] = it.grp_list[(int64_t)h * N + base + e];
      __syncthreads();
    } else {
      __shared__ uint16_t s_tmp[kUpdWindow];
      // thread tid holds the labels of window tokens tid*32 .. tid*32 + 31,
      // fetched as dwords when the head's labels are 4-byte aligned (N % 4 == 0)
      uint32_t kk[kUpdWindow / 256];
      {
        const int i0 = t0 + tid * 32;
        if ((N & 3) == 0 && i0 + 32 <= N) {
          uint32_t wv[8];
          const uint32_t* l4 = reinterpret_cast<const uint32_t*>(lab + i0);
  #pragma unroll
          for (int q = 0; q < 8; ++q) wv[q] = l4[q];
  #pragma unroll
          for (int x = 0; x < 32; ++x) kk[x] = ((wv[x >> 2] >> (8 * (x & 3))) & 0xFFu) - (uint32_t)c0;
        } else {
  #pragma unroll
          for (int x = 0; x < 32; ++x) {
            const int i = i0 + x;
            const uint32_t l = lab[min(i, N - 1)];                      // unconditional: one batch of loads
            kk[x] = i < N ? l - (uint32_t)c0 : 0xFFFFFFFFu;             // unsigned: in the group iff < 8
          }
        }
      }
      // (1) compact the window's members of the group into s_tmp (token << 3 |
      // cluster): per wave one ballot per label slot, the wave's range from the
      // wave totals (no atomics);  (2) counting sort of s_tmp by cluster into s_mem.
      int wtot = 0;
  #pragma unroll
      for (int x = 0; x < kUpdWindow / 256; ++x) wtot += __popcll(__ballot(kk[x] < (uint32_t)kUpdClusters));
      if (lane == 0) s_wtot[wave] = wtot;
      if (tid < kUpdClusters) s_cnt[tid] = 0;
      __syncthreads();
      int run = 0;
      for (int v = 0; v < wave; ++v) run += s_wtot[v];
      const int n_mem = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
  #pragma unroll
      for (int x = 0; x < kUpdWindow / 256; ++x) {
        const bool in = kk[x] < (uint32_t)kUpdClusters;
        const uint64_t m = __ballot(in);
        if (in) {
          const int pos = run + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          s_tmp[pos] = (uint16_t)(((tid * 32 + x) << 3) | kk[x]);
        }
        run += __popcll(m);
      }
      __syncthreads();
      for (int e = tid; e < n_mem; e += 256) atomicAdd(&s_cnt[s_tmp[e] & 7], 1);
      __syncthreads();
      if (tid == 0) {
        int a = 0;
        for (int k = 0; k < kUpdClusters; ++k) {
          s_off[k] = a;
          s_cur[k] = a;
          a += s_cnt[k];
        }
        s_off[kUpdClusters] = a;
      }
      __syncthreads();
      for (int e = tid; e < n_mem; e += 256) {
        const uint32_t v = s_tmp[e];
        s_mem[atomicAdd(&s_cur[v & 7], 1)] = (uint16_t)(v >> 3);
      }
      __syncthreads();
    }
    for (int sr = 0; sr < CPG / kUpdClusters; ++sr) {
    // pair p = 4 sr + w: clusters 2p and 2p + 1, member rows [ma, mb) and [mb, mc) of the list
    const int p = sr * 4 + wave;
    const int ma = s_off[p * 2], mb = s_off[p * 2 + 1], mc = s_off[p * 2 + 2];
    total[0] += mb - ma;
    total[1] += mc - mb;
    if (plain) {
      // Lane group g = lane / 32 sums cluster 2w + g alone, 8 bytes per lane
      // (channels c4 .. c4 + 3), kUpdRows of its member rows in flight: no
      // per-row selects and no join across the groups.  Float64 sums, exact
      // under the certificate.  A group whose cluster has fewer rows reads
      // clamped list entries (inside this window's list, which holds at least
      // one row whenever the loop runs) and adds nothing.
      const int g = lane >> 5, c4 = (lane & 31) * 4;
      const int64_t hoff4 = (int64_t)h * y.stride_head + c4;
      const int mg0 = g == 0 ? ma : mb, ng = g == 0 ? mb - ma : mc - mb;
      const int nmax = max(mb - ma, mc - mb);
      double sv[4];
      int64_t fv[4] = {0, 0, 0, 0};              // record_fix: integer sums in the head's units
      int em[4] = {1, 1, 1, 1};
      if (record_fix) {
#pragma unroll
        for (int e = 0; e < 4; ++e) em[e] = chan_emin(it, h, c4 + e);
      }
      u16x2 mx[2], mn[2];                        // magnitudes: max, and min nonzero - 1
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = 0.0;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        mx[p] = u16x2{0, 0};
        mn[p] = u16x2{0xFFFF, 0xFFFF};
      }
      for (int m = 0; m < nmax; m += kUpdRows) {
        uint2 raw[kUpdRows];
#pragma unroll
        for (int q = 0; q < kUpdRows; ++q) {
          const int r = max(mg0 + min(m + q, ng - 1), 0);
          raw[q] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(y.ptr) +
                                                   (int64_t)(t0 + s_mem[r]) * y.stride_token + hoff4);
        }
#pragma unroll
        for (int q = 0; q < kUpdRows; ++q) {
          if (m + q < ng) {
            const uint32_t w2[2] = {raw[q].x, raw[q].y};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              sv[2 * p] += (double)bf16_bits_to_f32(w2[p] & 0xFFFFu);
              sv[2 * p + 1] += (double)bf16_bits_to_f32(w2[p] >> 16);
              if (record_fix) {                  // workgroup-uniform
                fv[2 * p] += fix_of(w2[p] & 0xFFFFu, em[2 * p]);
                fv[2 * p + 1] += fix_of(w2[p] >> 16, em[2 * p + 1]);
              }
              const u16x2 mag = __builtin_bit_cast(u16x2, w2[p] & 0x7FFF7FFFu);
              mx[p] = __builtin_elementwise_max(mx[p], mag);
              mn[p] = __builtin_elementwise_min(mn[p], mag - u16x2{1, 1});   // a zero wraps to 0xFFFF
            }
          }
        }
      }
      // certificate of each group's cluster over its 32 lanes' channels
      bool ok;
      {
        const int lg = 32 - __builtin_clz((unsigned)max(ng, 1));   // >= ceil(log2 n)
        ok = true;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int emax = (int)(mx[p][e] >> 7), nz = (int)mn[p][e] + 1;      // nz: smallest nonzero magnitude
            const int emin = max((nz >> 7) & 0xFF, 1);                           // subnormals share exponent 1's unit
            ok = ok && (mn[p][e] == 0xFFFF || (emax < 0xFF && emax - emin + lg <= 44));
          }
      }
      const uint64_t bad = __ballot(!ok);
      const bool okc[2] = {(uint32_t)bad == 0u, (uint32_t)(bad >> 32) == 0u};
      if (record) {                              // the head's magnitude range (both clusters of the wave)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int k = c4 + 2 * p + e;
            if (mx[p][e]) atomicMax(&s_emag[0][k], (uint32_t)mx[p][e]);
            if (mn[p][e] != 0xFFFF) atomicMax(&s_emag[1][k], 0xFFFFu - (uint32_t)mn[p][e]);
          }
      }
      // certified clusters: lane group 0 finishes the first, group 1 the second
      {
        const int cc = g;
        const int n = cc == 0 ? mb - ma : mc - mb;
        const int j = c0 + p * 2 + cc;
        if (record && j < C) {                   // exact sums and counts for the incremental updates
          if (okc[cc]) {
            double2* ds = reinterpret_cast<double2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
            ds[0] = make_double2(sv[0], sv[1]);
            ds[1] = make_double2(sv[2], sv[3]);
          }
          if ((lane & 31) == 0) it.dcnt[h * C + j] = n;
        }
        if (record_fix && j < C) {               // the fixed-point head's integer sums (same storage)
          longlong2* ds = reinterpret_cast<longlong2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
          ds[0] = make_longlong2(fv[0], fv[1]);
          ds[1] = make_longlong2(fv[2], fv[3]);
          if ((lane & 31) == 0) it.dcnt[h * C + j] = n;
        }
        if (okc[cc] && n > 0 && j < C) centroid_from_sum(it, h, C, j, c4, sv, n);
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        old_fin[cc] = !okc[cc];
        if (!okc[cc]) {                             // rare: this cluster again in double-double
          const int m0 = cc == 0 ? ma : mb, m1 = cc == 0 ? mb : mc;
          dd_rows(t0, m0, m1, acc[cc][0], acc[cc][1]);
        }
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) dd_rows(t0, cc == 0 ? ma : mb, cc == 0 ? mb : mc, acc[cc][0], acc[cc][1]);
    }
    if constexpr (GROUPED) {                   // one window: this pair is complete
      finish_pair(p);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        acc[cc][0] = DD{0.0, 0.0};
        acc[cc][1] = DD{0.0, 0.0};
        total[cc] = 0;
        old_fin[cc] = true;
      }
    }
    }
    __syncthreads();                           // the lists are rebuilt for the next window
  }
  if constexpr (!GROUPED) finish_pair(wave);
  if (record) {                                  // this workgroup's clusters into the head's range
    const uint32_t v = s_emag[tid >> 7][tid & (kHeadDim - 1)];
    if (v) atomicMax(&it.emag[((int64_t)h * 2 + (tid >> 7)) * kHeadDim + (tid & (kHeadDim - 1))], v);
  }
}

template <bool F32, bool GROUPED, int CPG>
__global__ __launch_bounds__(256, 4) void k_update(KmBatch b) {
  const int groups = (b.C + CPG - 1) / CPG;
  const uint32_t logical = xcd_remap(blockIdx.x, (uint32_t)(b.H * groups));
  const KmItem& it = b.it[blockIdx.y];
  if (blockIdx.x == 0 && threadIdx.x == 0 && it.amb_count) *it.amb_count = 0;   // the next assign's close calls
  update_block<F32, GROUPED, CPG>(b, blockIdx.y, logical / groups, (logical % groups) * CPG);
}

// The full update of the listed heads (bf16 tokens, grouped, inc == 2).
template <int CPG>
__global__ __launch_bounds__(256, 4) void k_update_list(KmBatch b) {
  const int groups = (b.C + CPG - 1) / CPG;
  if (blockIdx.x == 0 && threadIdx.x < b.n && b.it[threadIdx.x].amb_count) *b.it[threadIdx.x].amb_count = 0;
  __shared__ int s_n[kKmMaxBatch];
  listed_counts(b, groups, s_n);
  int e = blockIdx.x;
  for (int p = 0; p < b.n; ++p) {
    const KmItem& it = b.it[p];
    const int cnt = s_n[p];
    for (; e < cnt; e += gridDim.x) {
      update_block<false, true, CPG>(b, p, listed_head(b, it, e / groups), (e % groups) * CPG);
      __syncthreads();                           // the LDS lists are rebuilt for the next item
    }
    e -= cnt;
  }
}

// Incremental update (the iterations after the first of a stage, bf16 heads
// that pass head_exact): kDeltaSplit workgroups per (problem, head).  Each
// scans the head's labels against those of the previous update, counts the
// tokens that moved into and out of every cluster and lists them by cluster in
// LDS (counting sort); the touched clusters, in index order, are dealt
// round-robin to the workgroups and then to their eight 32-lane groups.  A
// lane group (four channels per lane) adds its cluster's arriving rows to the
// kept float64 sum and subtracts the leaving ones -- exact under the
// certificate, so the order is free and the sum equals the full update's --
// updates the member count and forms the centroid with centroid_from_sum; a
// cluster left empty keeps its centroid.  The workgroup of split 0 also copies
// the current labels into the other alternate buffer, where the next update
// finds them as its previous labels.
constexpr int kDeltaSplit = 2;
constexpr int kDeltaSlots = 2;               // clusters per lane group in flight
constexpr int kDeltaRows = 4;                 // member-row loads in flight per cluster

__global__ __launch_bounds__(256) void k_update_delta(KmBatch b) {
  const KmItem& it = b.it[blockIdx.y];
  const int C = b.C, N = (int)b.N, n_heads = b.H;
  const uint32_t logical = xcd_remap(blockIdx.x, (uint32_t)(n_heads * kDeltaSplit));
  const int h = logical / kDeltaSplit, r = logical % kDeltaSplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t cert = it.cert[h];
  if (cert == 0 || (cert == kCertFix && b.iter < 2)) return;   // the full update took this head
  const bool fixp = cert == kCertFix;            // integer sums in the head's units
  __shared__ int s_cnt[256], s_off[257], s_cur[256];
  __shared__ uint16_t s_item[2 * kUpdWindow];    // token, | 0x8000 when it leaves the cluster
  __shared__ uint8_t s_touch[256];
  __shared__ int s_nt;
  const uint8_t* cur = it.labels + (int64_t)h * N;
  const uint8_t* prv = it.prev + ((int64_t)(b.iter & 1) * n_heads + h) * N;
  uint8_t* nxt = it.prev + ((int64_t)((b.iter + 1) & 1) * n_heads + h) * N;
  uint32_t kc[kUpdWindow / 256], kp[kUpdWindow / 256];   // labels of tokens tid*32 .. tid*32 + 31: now, before
  {
    const int i0 = tid * 32;
    if ((N & 3) == 0 && i0 + 32 <= N) {
      uint32_t wc[8], wp[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        wc[q] = reinterpret_cast<const uint32_t*>(cur + i0)[q];
        wp[q] = reinterpret_cast<const uint32_t*>(prv + i0)[q];
      }
      if (r == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) reinterpret_cast<uint32_t*>(nxt + i0)[q] = wc[q];
      }
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        kc[x] = (wc[x >> 2] >> (8 * (x & 3))) & 0xFFu;
        kp[x] = (wp[x >> 2] >> (8 * (x & 3))) & 0xFFu;
      }
    } else {
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        const int i = i0 + x;
        const uint32_t lc = cur[min(i, N - 1)], lp = prv[min(i, N - 1)];
        kc[x] = i < N ? lc : 0u;                 // past the head: no move
        kp[x] = i < N ? lp : 0u;
        if (r == 0 && i < N) nxt[i] = (uint8_t)lc;
      }
    }
  }
  s_cnt[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 32; ++x)
    if (kc[x] != kp[x]) {
      atomicAdd(&s_cnt[kc[x]], 1);
      atomicAdd(&s_cnt[kp[x]], 1);
    }
  __syncthreads();
  if (wave == 0) {                               // exclusive prefix (four clusters per lane) and the touched list
    int a[4], sum = 0, nz = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = s_cnt[lane * 4 + e];
      sum += a[e];
      nz += a[e] > 0 ? 1 : 0;
    }
    int incl = sum, tincl = nz;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o), tt = __shfl_up(tincl, o);
      if (lane >= o) {
        incl += t;
        tincl += tt;
      }
    }
    int ex = incl - sum, tp = tincl - nz;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_off[lane * 4 + e] = ex;
      s_cur[lane * 4 + e] = ex;
      ex += a[e];
      if (a[e] > 0) s_touch[tp++] = (uint8_t)(lane * 4 + e);
    }
    if (lane == 63) {
      s_off[256] = incl;
      s_nt = tincl;
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 32; ++x)
    if (kc[x] != kp[x]) {
      const int tok = tid * 32 + x;
      s_item[atomicAdd(&s_cur[kp[x]], 1)] = (uint16_t)(tok | 0x8000);
      s_item[atomicAdd(&s_cur[kc[x]], 1)] = (uint16_t)tok;
    }
  __syncthreads();
  const int nt = s_nt;
  const int g = lane >> 5, c4 = (lane & 31) * 4;
  int em[4] = {1, 1, 1, 1};
  if (fixp) {
#pragma unroll
    for (int e = 0; e < 4; ++e) em[e] = chan_emin(it, h, c4 + e);
  }
  const uint16_t* y16 = reinterpret_cast<const uint16_t*>(it.y);
  const int64_t hoff4 = (int64_t)h * it.stride_head + c4;
  // Lane group lg = 2 * wave + g takes the touched clusters q = r + kDeltaSplit * (lg + 8 k),
  // kDeltaSlots of them at a time, so that the loads of several clusters (their
  // sums, counts and member rows) are in flight together.
  const int lg = 2 * wave + g;
  for (int base = r + kDeltaSplit * lg; base < nt; base += kDeltaSplit * 8 * kDeltaSlots) {
    int jj[kDeltaSlots], i0[kDeltaSlots], ni[kDeltaSlots], n_old[kDeltaSlots], dn[kDeltaSlots];
    bool mine[kDeltaSlots];
    double sv[kDeltaSlots][4];
    int64_t fv[kDeltaSlots][4];
    int nmax = 0;
#pragma unroll
    for (int sl = 0; sl < kDeltaSlots; ++sl) {
      const int q = base + sl * kDeltaSplit * 8;
      const bool live = q < nt;
      const int j = live ? (int)s_touch[q] : 0;
      jj[sl] = j;
      i0[sl] = live ? s_off[j] : 0;
      ni[sl] = live ? s_cnt[j] : 0;
      dn[sl] = 0;
      nmax = max(nmax, ni[sl]);
      mine[sl] = live && j < C;
      n_old[sl] = mine[sl] ? it.dcnt[h * C + j] : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[sl][e] = 0.0;
        fv[sl][e] = 0;
      }
      if (mine[sl] && fixp) {
        const longlong2* ds = reinterpret_cast<const longlong2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
        const longlong2 d0 = ds[0], d1 = ds[1];
        fv[sl][0] = d0.x;
        fv[sl][1] = d0.y;
        fv[sl][2] = d1.x;
        fv[sl][3] = d1.y;
      } else if (mine[sl]) {
        const double2* ds = reinterpret_cast<const double2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
        const double2 d0 = ds[0], d1 = ds[1];
        sv[sl][0] = d0.x;
        sv[sl][1] = d0.y;
        sv[sl][2] = d1.x;
        sv[sl][3] = d1.y;
      }
    }
    nmax = max(nmax, __shfl_xor(nmax, 32));
    for (int m = 0; m < nmax; m += kDeltaRows) {
      uint32_t itm[kDeltaSlots][kDeltaRows];
      uint2 raw[kDeltaSlots][kDeltaRows];
#pragma unroll
      for (int sl = 0; sl < kDeltaSlots; ++sl) {
#pragma unroll
        for (int q2 = 0; q2 < kDeltaRows; ++q2) {   // past a cluster's items: loaded, not added
          itm[sl][q2] = s_item[i0[sl] + min(m + q2, max(ni[sl] - 1, 0))];
          raw[sl][q2] =
              *reinterpret_cast<const uint2*>(y16 + (int64_t)(itm[sl][q2] & 0x7FFFu) * it.stride_token + hoff4);
        }
      }
#pragma unroll
      for (int sl = 0; sl < kDeltaSlots; ++sl) {
#pragma unroll
        for (int q2 = 0; q2 < kDeltaRows; ++q2) {
          if (m + q2 < ni[sl]) {
            const bool out = (itm[sl][q2] & 0x8000u) != 0;
            const uint32_t w2[2] = {raw[sl][q2].x, raw[sl][q2].y};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              if (fixp) {                        // workgroup-uniform
                const int64_t f0 = fix_of(w2[p] & 0xFFFFu, em[2 * p]), f1 = fix_of(w2[p] >> 16, em[2 * p + 1]);
                fv[sl][2 * p] = out ? fv[sl][2 * p] - f0 : fv[sl][2 * p] + f0;
                fv[sl][2 * p + 1] = out ? fv[sl][2 * p + 1] - f1 : fv[sl][2 * p + 1] + f1;
              } else {
                const double v0 = (double)bf16_bits_to_f32(w2[p] & 0xFFFFu);
                const double v1 = (double)bf16_bits_to_f32(w2[p] >> 16);
                sv[sl][2 * p] = out ? sv[sl][2 * p] - v0 : sv[sl][2 * p] + v0;
                sv[sl][2 * p + 1] = out ? sv[sl][2 * p + 1] - v1 : sv[sl][2 * p + 1] + v1;
              }
            }
            dn[sl] += out ? -1 : 1;
          }
        }
      }
    }
#pragma unroll
    for (int sl = 0; sl < kDeltaSlots; ++sl) {
      if (!mine[sl]) continue;
      const int j = jj[sl], n = n_old[sl] + dn[sl];
      if (fixp) {
        longlong2* ds = reinterpret_cast<longlong2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
        ds[0] = make_longlong2(fv[sl][0], fv[sl][1]);
        ds[1] = make_longlong2(fv[sl][2], fv[sl][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[sl][e] = fix_to_f64(fv[sl][e], em[e]);   // the exact sum, rounded once
      } else {
        double2* ds = reinterpret_cast<double2*>(it.dsum + ((int64_t)h * C + j) * kHeadDim + c4);
        ds[0] = make_double2(sv[sl][0], sv[sl][1]);
        ds[1] = make_double2(sv[sl][2], sv[sl][3]);
      }
      if ((lane & 31) == 0) it.dcnt[h * C + j] = n;
      if (n > 0) centroid_from_sum(it, h, C, j, c4, sv[sl], n);
    }
  }
}

// cert[h], the head's class, for every head of every problem (one wave per head);
// the heads outside the float64 class are appended to the problem's hlist.
__global__ __launch_bounds__(64) void k_cert(KmBatch b) {
  const KmItem& it = b.it[blockIdx.y];
  const int h = blockIdx.x;
  const bool f64 = head_span_ok(it, h, (int)b.N, 44), fix = head_span_ok(it, h, (int)b.N, 55);
  if (threadIdx.x == 0) {
    const uint32_t cl = f64 ? kCertF64 : fix ? kCertFix : 0u;
    it.cert[h] = cl;
    if (cl != kCertF64) {                        // the later full updates' head lists
      const int k = cl == kCertFix ? 1 : 0;
      const uint32_t slot = atomicAdd(&it.hlist[k], 1u);   // one entry per head: slot < H
      if (slot < (uint32_t)b.H) it.hlist[2 + k * b.H + slot] = (uint32_t)h;
    }
  }
}

// Eight values per thread (H * C * 128 is a multiple of 8; both tables are
// 16-byte aligned): two 16-byte loads, one 16-byte store.
__global__ void k_centroid_bf16(KmBatch b) {
  const KmItem& it = b.it[blockIdx.y];
  const int64_t n8 = (int64_t)b.H * b.C * (kHeadDim / 8);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(it.c)[2 * i];
  const float4 c = reinterpret_cast<const float4*>(it.c)[2 * i + 1];
  uint4 o;
  o.x = f32_to_bf16_bits(a.x) | (f32_to_bf16_bits(a.y) << 16);
  o.y = f32_to_bf16_bits(a.z) | (f32_to_bf16_bits(a.w) << 16);
  o.z = f32_to_bf16_bits(c.x) | (f32_to_bf16_bits(c.y) << 16);
  o.w = f32_to_bf16_bits(c.z) | (f32_to_bf16_bits(c.w) << 16);
  reinterpret_cast<uint4*>(it.cent_bf16)[i] = o;
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_kmeans_init(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_init", s);
  const dim3 grid((b.C + 7) / 8, b.H, b.n);
  if (b.dtype == 0) hipLaunchKernelGGL(k_init<true>, grid, dim3(256), 0, s, b);
  else hipLaunchKernelGGL(k_init<false>, grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_kmeans_assign(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_assign", s);
  if (b.C > kAsgMaxC) return hipErrorInvalidValue;
  // Workgroups per head G: each workgroup pays a fixed cost (plane load,
  // first tokens, close calls; about kAsgUnitCost sub-blocks' worth) and the
  // launch runs in rounds of one workgroup per compute unit, so G minimizes
  // rounds x (sub-blocks per workgroup + fixed cost).
  const int S = (int)((b.N + 31) / 32);
  int G = 1;
  double best = 1e300;
  for (int g = 1; g <= std::min(S, 64); ++g) {
    const int64_t rounds = ((int64_t)b.n * b.H * g + kAsgCUs - 1) / kAsgCUs;
    const double cost = (double)rounds * ((S + g - 1) / g + kAsgUnitCost);
    if (cost < best) {
      best = cost;
      G = g;
    }
  }
  const dim3 grid((unsigned)(G * b.H), b.n);
  if (b.dtype == 0) hipLaunchKernelGGL(k_assign<true>, grid, dim3(kAsgThreads), 0, s, b, G);
  else hipLaunchKernelGGL(k_assign<false>, grid, dim3(kAsgThreads), 0, s, b, G);
  return hipGetLastError();
}

hipError_t launch_kmeans_update(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_update", s);
  const bool grouped = b.it[0].grp_off != nullptr && b.N <= kUpdWindow;   // set for all problems or none
  // 32 clusters per workgroup when the launch holds enough work to fill the
  // chip with the fewer, longer workgroups (measured: 7 % faster at 12
  // problems of 32 heads, 10 % slower at 2)
  // Incremental iterations (inc == 2) take only the heads k_cert listed: in the
  // first, the fixed-point heads on the shorter 8-cluster workgroups (few heads,
  // more workgroups each); later the heads outside both classes, usually none.
  if (b.inc == 2) {                              // the listed heads: fixed-point ones once, then the rest
    if (!grouped || b.dtype != 1 || !b.it[0].hlist) return hipErrorInvalidValue;
    const int cpg = b.iter == 1 ? kUpdClusters : kUpdClustersG;
    const int64_t items = (int64_t)b.n * b.H * ((b.C + cpg - 1) / cpg);
    const dim3 grid((unsigned)std::min<int64_t>(items, kListUpdateGrid));
    if (b.iter == 1) hipLaunchKernelGGL(k_update_list<kUpdClusters>, grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL(k_update_list<kUpdClustersG>, grid, dim3(256), 0, s, b);
    return hipGetLastError();
  }
  const bool wide = grouped && (int64_t)b.n * b.H * b.C >= 6 * 32 * 256;
  const int cpg = wide ? kUpdClustersG : kUpdClusters;
  const dim3 grid((unsigned)(b.H * ((b.C + cpg - 1) / cpg)), b.n);
  if (wide) {
    if (b.dtype == 0) hipLaunchKernelGGL((k_update<true, true, kUpdClustersG>), grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((k_update<false, true, kUpdClustersG>), grid, dim3(256), 0, s, b);
  } else if (grouped) {
    if (b.dtype == 0) hipLaunchKernelGGL((k_update<true, true, kUpdClusters>), grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((k_update<false, true, kUpdClusters>), grid, dim3(256), 0, s, b);
  } else {
    if (b.dtype == 0) hipLaunchKernelGGL((k_update<true, false, kUpdClusters>), grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((k_update<false, false, kUpdClusters>), grid, dim3(256), 0, s, b);
  }
  return hipGetLastError();
}

hipError_t launch_kmeans_update_delta(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_update_delta", s);
  if (b.inc != 2 || b.dtype != 1 || b.N > kUpdWindow || b.C > 256 || !b.it[0].dsum) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(b.H * kDeltaSplit), b.n);
  hipLaunchKernelGGL(k_update_delta, grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_kmeans_cert(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_cert", s);
  if (b.inc != 1 || !b.it[0].cert) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cert, dim3(b.H, b.n), dim3(64), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_kmeans_group(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_group", s);
  if (b.N > kUpdWindow || b.C > 256) return hipErrorInvalidValue;
  if (b.inc == 2) {                              // the listed heads only
    if (!b.it[0].hlist) return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>((int64_t)b.n * b.H, kListGroupGrid));
    hipLaunchKernelGGL(k_group_list, grid, dim3(256), 0, s, b);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_group, dim3(b.H, b.n), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_centroid_bf16(const KmBatch& b, hipStream_t s) {
  TimedLaunch tl_("k_centroid_bf16", s);
  const int64_t n8 = (int64_t)b.H * b.C * (kHeadDim / 8);
  hipLaunchKernelGGL(k_centroid_bf16, dim3((unsigned)((n8 + 255) / 256), b.n), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u32(void* p, size_t n_words, hipStream_t s) {
  TimedLaunch tl_("k_fill_zero", s);
  if (n_words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), (int64_t)n_words);
  return hipGetLastError();
}

}  // namespace qkv
