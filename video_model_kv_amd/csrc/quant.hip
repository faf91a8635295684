// Residual, per-group scale, rounding and bit packing of one stage; and the
// inverse (dequantization), and the PSAC coefficient encoder.
//
// Method: Quant VideoGen notes, "Research background / core tension" (symmetric
// per-group quantization, S = max|X| / (2^(b-1) - 1), X_INT = round(X / S)) and
// "Method / Overall framework" (residual against the token's centroid, BF16
// centroids, dequantization S * X_INT + C_i); mixed 4/2-bit classes from the
// 2-bit trap explainer (section five, advice one) and the practitioner blog
// (section 3.2); PSAC coefficients from the QuantWM summary ("QuantWM", second
// technique).
//
// Arithmetic (matches the documented format bit for bit):
//   r = fp32(y - C_bf16[label]);  S = bf16_rne(fp32(max|r| / qmax));
//   q = S == 0 ? 0 : clamp(rint_even(fp32(r / S)), -2^(b-1), 2^(b-1) - 1);
//   y_hat = fp32(S * q + C) (S * q is exact);  y_next = fp32(y - y_hat).
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

struct GroupInfo {
  int start;      // first storage position (index into the perm order)
  int len;        // channels in the group
  int bits;
  int pos0;       // position of the first channel within its class
  int word0;      // first word of the class
};

// Group g (storage order) of the uniform or mixed layout.
__device__ __forceinline__ GroupInfo group_info(int g, int bits, int group, int n_int4, int int4_words) {
  GroupInfo gi;
  if (n_int4 > 0) {
    const int g4 = (n_int4 + group - 1) / group;
    if (g < g4) {
      gi.pos0 = g * group;
      gi.len = min(group, n_int4 - gi.pos0);
      gi.bits = 4;
      gi.word0 = 0;
      gi.start = gi.pos0;
    } else {
      gi.pos0 = (g - g4) * group;
      gi.len = min(group, kHeadDim - n_int4 - gi.pos0);
      gi.bits = bits;
      gi.word0 = int4_words;
      gi.start = n_int4 + gi.pos0;
    }
  } else {
    gi.pos0 = g * group;
    gi.len = group;
    gi.bits = bits;
    gi.word0 = 0;
    gi.start = gi.pos0;
  }
  return gi;
}

// Decode entry of the channel at storage position p.
__device__ __forceinline__ ChannelCode code_of(int p, int bits, int group, int n_int4, int int4_words) {
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

template <bool F32>
__device__ __forceinline__ float load_y(const TensorView& y, int64_t tok, int h, int k) {
  const int64_t off = tok * y.stride_token + (int64_t)h * y.stride_head + k;
  if constexpr (F32) return reinterpret_cast<const float*>(y.ptr)[off];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(y.ptr)[off]);
}

// Codes of NE residuals of one group by the definition: q_e =
// clamp(rint(fp32(r_e / S))) with the correctly rounded division; S == 0
// gives q = 0.
template <int NE>
__device__ __forceinline__ void group_codes(const float* r, float S, float qlo, float qhi, float* q) {
#pragma unroll
  for (int e = 0; e < NE; ++e) q[e] = S != 0.0f ? __builtin_amdgcn_fmed3f(rintf(r[e] / S), qlo, qhi) : 0.0f;
}

// DPP lane exchanges inside a row of 16 lanes (all lanes active): quad_perm
// swaps for xor 1 and xor 2, then half-row and row mirrors, which pair every
// lane of one aligned half with a lane of the other half.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int LANES>   // max over aligned groups of LANES lanes (1, 2, 4, 8 or 16)
__device__ __forceinline__ float group_max_dpp(float v) {
  if constexpr (LANES >= 2) v = fmaxf(v, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v))));   // [1,0,3,2]
  if constexpr (LANES >= 4) v = fmaxf(v, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v))));   // [2,3,0,1]
  if constexpr (LANES >= 8) v = fmaxf(v, __uint_as_float(dpp_u32<0x141>(__float_as_uint(v))));  // half mirror
  if constexpr (LANES >= 16) v = fmaxf(v, __uint_as_float(dpp_u32<0x140>(__float_as_uint(v))));  // mirror
  return v;
}

// Stored codes u = q + 2^(b-1) of 8 residuals sharing the scale S (bits
// S_bits), packed b bits per channel; the arithmetic of group_codes with
// shortcuts that do not change a result:
//  * fp32(1 / S) is read from a table of fp32(1 / m) over the 128 bf16
//    significands m, scaled by the exponent (exact for normal S);
//  * one refinement step suffices: with x = r / S, q0 = fp32(r * rS) is within
//    1.5 ulp(x), the remainder e = r - q0 S is exact, and the fused step
//    fp32(q0 + e * rS) = fp32(x + eta) with |eta| < 1.5 * 2^-24 ulp(x).  As S
//    has an 8-bit significand, x is never a rounding midpoint and lies at
//    least ulp(x) / 512 away from every midpoint, so the step rounds like x;
//  * rint and the offset come from one addition of 1.5 * 2^23 + 2^(b-1)
//    (round to nearest even at unit spacing);
//  * the clamp is dropped, since |r| <= max|r| <= qmax * S * (1 + 2^-8.9)
//    keeps |q| <= qmax.
// Scales outside [2^-96, 2^96] (and S == 0) take group_codes.
template <int BITS>
__device__ __forceinline__ uint32_t pack8_codes(const float* r, float S, uint32_t S_bits, const float* rtab) {
  constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
  const uint32_t E = (S_bits >> 7) & 0xFFu;
  uint32_t w = 0;
  if (__builtin_expect(E >= 31u && E <= 223u, 1)) {            // S in [2^-96, 2^96)
    const float rS = __builtin_amdgcn_ldexpf(rtab[S_bits & 0x7Fu], 127 - (int)E);
    constexpr float kBias = 12582912.0f + (float)(1 << (BITS - 1));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = r[e] * rS;
      x = __builtin_fmaf(__builtin_fmaf(-x, S, r[e]), rS, x);
      const uint32_t z = __float_as_uint(x + kBias);           // 0x4B400000 + u, u < 2^BITS
      // INT2: bits 2..21 of z are zero, so z << 2e carries u at bits [2e, 2e + 2)
      // and nothing else below bit 22; the word is cut to 16 bits at the end
      if constexpr (BITS == 2) w |= z << (BITS * e);
      else w |= (z & ((1u << BITS) - 1u)) << (BITS * e);
    }
    if constexpr (BITS == 2) w &= 0xFFFFu;
  } else {
    float q[8];
    group_codes<8>(r, S, -(float)(1 << (BITS - 1)), qmax, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= (uint32_t)((int)q[e] + (1 << (BITS - 1))) << (BITS * e);
  }
  return w;
}

// One thread per (head, token, group).
template <int G, bool F32>
__global__ __launch_bounds__(256) void k_quant_pack(PackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.H * a.N * a.groups;
  if (gid >= total) return;
  const int g = (int)(gid % a.groups);
  const int64_t t = gid / a.groups;
  const int i = (int)(t % a.N);
  const int h = (int)(t / a.N);
  const GroupInfo gi = group_info(g, a.bits, a.group, a.n_int4, a.int4_words);
  const int lab = min((int)a.labels[(int64_t)h * a.N + i], a.C - 1);   // labels < C (memory safety)
  const uint16_t* crow = a.centroids + ((int64_t)h * a.C + lab) * kHeadDim;
  const uint8_t* perm = a.perm ? a.perm + h * kHeadDim : nullptr;

  float r[G];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    r[e] = 0.0f;
    if (e < gi.len) {
      const int p = gi.start + e;
      const int k = perm ? (perm[p] & (kHeadDim - 1)) : p;
      const float yv = load_y<F32>(a.y, i, h, k);
      const float cv = bf16_bits_to_f32(crow[k]);
      r[e] = yv - cv;
      amax = fmaxf(amax, fabsf(r[e]));
    }
  }
  const int b = gi.bits;
  const float qmax = (float)((1 << (b - 1)) - 1);
  const uint32_t sbits = f32_to_bf16_bits(amax / qmax);
  const float S = bf16_bits_to_f32(sbits);
  const float qlo = -(float)(1 << (b - 1)), qhi = qmax;
  const int per = 32 / b;
  const uint32_t off = 1u << (b - 1);
  uint32_t words[G / 8];
#pragma unroll
  for (int w = 0; w < G / 8; ++w) words[w] = 0u;
  const int64_t ynext_base = ((int64_t)h * a.N + i) * kHeadDim;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    if (e < gi.len) {
      float q = 0.0f;
      if (S != 0.0f) q = fminf(fmaxf(rintf(r[e] / S), qlo), qhi);
      const uint32_t u = (uint32_t)((int)q + (int)off);
      const int pc = gi.pos0 + e;            // position in class
      const int wl = e / per;                // word within the group (pos0 is word aligned)
      words[wl] |= u << (b * (pc % per));
      if (a.y_next) {
        const int p = gi.start + e;
        const int k = perm ? (perm[p] & (kHeadDim - 1)) : p;
        const float yv = load_y<F32>(a.y, i, h, k);
        const float cv = bf16_bits_to_f32(crow[k]);
        const float yhat = __fadd_rn(S * q, cv);
        a.y_next[ynext_base + k] = __fsub_rn(yv, yhat);
      }
    }
  }
  const int nw = (gi.len + per - 1) / per;
  uint32_t* wout = a.codes + ((int64_t)h * a.N + i) * a.words + gi.word0 + gi.pos0 / per;
#pragma unroll
  for (int w = 0; w < G / 8; ++w)
    if (w < nw) wout[w] = words[w];
  a.scales[((int64_t)h * a.N + i) * a.groups + g] = (uint16_t)sbits;
}

// Uniform layout without a channel permutation.  A workgroup owns a tile of
// T tokens x HB heads (HB = min(H, 4), T * HB <= 64 rows) taken in
// token-major order: with the usual [N][H][128] input that is T runs of 1 KB
// (4 bf16 heads).  Tiles run head block by head block, so the workgroups an
// XCD holds at a time share a few heads' centroid tables in its L2 and read
// neighbouring token rows.  A thread handles 8 consecutive channels of a row
// (one 16-byte load) in each of 4 items; a wave covers 4 rows per item; a
// group of G channels spans G/8 aligned lanes and takes its max through DPP
// lane exchanges.  Codes and scales are staged in LDS and written per head as
// contiguous runs of T rows (512 B of INT2 codes).  Same results as
// k_quant_pack.
constexpr int kTileRows = 64;
struct TileGeom {
  int HB, T, nhb, tiles;    // heads per tile, tokens per tile, head blocks, tiles per problem
};
constexpr int kTileHeads = 4;
__host__ __device__ inline TileGeom tile_geom(int H, int N) {
  TileGeom g;
  g.HB = H < kTileHeads ? H : kTileHeads;
  g.T = kTileRows / g.HB;
  g.nhb = (H + g.HB - 1) / g.HB;
  g.tiles = ((N + g.T - 1) / g.T) * g.nhb;
  return g;
}

template <int G, int BITS, bool F32>
__global__ __launch_bounds__(256) void k_quant_pack_tile(PackBatch pb, int tiles) {
  constexpr int L = G / 8;                        // lanes per group
  constexpr int W = kHeadDim * BITS / 32;         // code words per row
  constexpr int NG = kHeadDim / G;                // groups per row
  constexpr int kIt = kTileRows * 16 / 256;       // items per thread
  __shared__ __attribute__((aligned(16))) uint32_t s_codes[kTileRows * W];
  __shared__ uint16_t s_scales[kTileRows * NG];
  __shared__ float s_rtab[128];                   // fp32(1 / (1 + k / 128))
  if (threadIdx.x < 128) s_rtab[threadIdx.x] = 1.0f / (1.0f + (float)threadIdx.x * 0.0078125f);
  __syncthreads();
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);   // consecutive tiles share an XCD (L2)
  const PackArgs& a = pb.a[logical / tiles];
  const int tile = (int)(logical % tiles);
  const TileGeom tg = tile_geom(a.H, a.N);
  const int ntb = (a.N + tg.T - 1) / tg.T;         // token blocks; tiles run head block by head block
  const int hb = tile / ntb;
  const int i0 = (tile % ntb) * tg.T, h0 = hb * tg.HB;
  const int rows = tg.T * tg.HB;                  // <= kTileRows
  const int tid = threadIdx.x;
  const int part = tid & 15, k0 = part * 8;
  // local row lr = x * 16 + tid / 16 of item x splits as lr = t * HB + hh;
  // t = (lr * inv) >> 16 is exact for lr < 128, HB <= 128 (here lr < 64)
  const uint32_t inv = 65536u / (uint32_t)tg.HB + 1u;
  auto split = [&](int x, int& t, int& hh) __attribute__((always_inline)) {
    const int lr = x * 16 + (tid >> 4);
    t = (int)(__umul24((uint32_t)lr, inv) >> 16);
    hh = lr - (int)__umul24((uint32_t)t, (uint32_t)tg.HB);
  };
  // Addresses: 64-bit tile bases (wave-uniform) plus 32-bit in-tile offsets
  // formed with 24-bit multiplies (the launcher routes strides or token
  // counts of 2^23 or more to k_quant_pack).  Rows outside the tile are
  // clamped to the last valid token and head.
  const int tmax = a.N - 1 - i0, hmax = a.H - 1 - h0;
  const uint32_t ST = (uint32_t)a.y.stride_token, SH = (uint32_t)a.y.stride_head, NN = (uint32_t)a.N;
  const uint8_t* lab_base = a.labels + (int64_t)h0 * a.N + i0;
  const uint16_t* cent_base = a.centroids + (int64_t)h0 * a.C * kHeadDim + k0;
  const int64_t y_base = (int64_t)i0 * a.y.stride_token + (int64_t)h0 * a.y.stride_head + k0;

  // Every load is unconditional (rows outside the tile read a clamped, valid
  // row and are never stored), so no branch separates them and all of a
  // thread's requests are in flight together: labels, then the input rows,
  // then the labelled centroid rows (the memory counter drains in order, so
  // the centroid requests wait on the labels only).
  uint32_t lab[kIt];
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    int t, hh;
    split(x, t, hh);
    lab[x] = lab_base[__umul24((uint32_t)min(hh, hmax), NN) + (uint32_t)min(t, tmax)];
  }
  uint32_t yw[kIt][F32 ? 8 : 4];
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    int t, hh;
    split(x, t, hh);
    const uint32_t yo = __umul24((uint32_t)min(t, tmax), ST) + __umul24((uint32_t)min(hh, hmax), SH);
    if constexpr (F32) {
      const float* p = reinterpret_cast<const float*>(a.y.ptr) + y_base + yo;
      const uint4 p0 = *reinterpret_cast<const uint4*>(p);
      const uint4 p1 = *reinterpret_cast<const uint4*>(p + 4);
      yw[x][0] = p0.x; yw[x][1] = p0.y; yw[x][2] = p0.z; yw[x][3] = p0.w;
      yw[x][4] = p1.x; yw[x][5] = p1.y; yw[x][6] = p1.z; yw[x][7] = p1.w;
    } else {
      const uint4 p = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.y.ptr) + y_base + yo);
      yw[x][0] = p.x; yw[x][1] = p.y; yw[x][2] = p.z; yw[x][3] = p.w;
    }
  }
  uint4 cw[kIt];
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    int t, hh;
    split(x, t, hh);
    const uint32_t row = __umul24((uint32_t)min(hh, hmax), (uint32_t)a.C) + (uint32_t)min((int)lab[x], a.C - 1);
    cw[x] = *reinterpret_cast<const uint4*>(cent_base + row * kHeadDim);
  }
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    const int lr = x * 16 + (tid >> 4);
    int t, hh;
    split(x, t, hh);
    const bool ok = lr < rows && hh <= hmax && t <= tmax;   // uniform over a row's 16 lanes
    float yv[8], cv[8], r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (F32) yv[e] = __uint_as_float(yw[x][e]);
      else yv[e] = bf16_bits_to_f32((yw[x][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
    const uint32_t c4[4] = {cw[x].x, cw[x].y, cw[x].z, cw[x].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) cv[e] = bf16_bits_to_f32((c4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      r[e] = yv[e] - cv[e];
      amax = fmaxf(amax, fabsf(r[e]));
    }
    amax = group_max_dpp<L>(amax);
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
    const uint32_t sbits = f32_to_bf16_bits(amax / qmax);
    const float S = bf16_bits_to_f32(sbits);
    const uint32_t bitsw = pack8_codes<BITS>(r, S, sbits, s_rtab);
    if constexpr (BITS == 2) {
      const uint32_t other = dpp_u32<0xB1>(bitsw);
      if ((part & 1) == 0) s_codes[lr * W + (part >> 1)] = bitsw | (other << 16);
    } else {
      s_codes[lr * W + part] = bitsw;
    }
    if (part % L == 0) s_scales[lr * NG + part / L] = (uint16_t)sbits;
    if (ok && a.y_next) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = (float)((int)((bitsw >> (BITS * e)) & ((1u << BITS) - 1u)) - (1 << (BITS - 1)));
        o[e] = __fsub_rn(yv[e], __fadd_rn(S * q, cv[e]));
      }
      float* yp = a.y_next + ((int64_t)(h0 + hh) * a.N + i0 + t) * kHeadDim + k0;
      *reinterpret_cast<float4*>(yp) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(yp + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
  __syncthreads();
  // write-out: per head, the tile's T rows are contiguous in [H][N] order;
  // n / d for n, d <= 1024 as (n * (2^20 / d + 1)) >> 20 (exact there)
  const int tv = min(tg.T, a.N - i0);             // valid tokens of the tile
  constexpr int W4 = W / 4;
  {
    const uint32_t d = (uint32_t)tg.T * W4, dinv = (1u << 20) / d + 1u;
    uint32_t* cbase = a.codes + ((int64_t)h0 * a.N + i0) * W;
    for (int idx = tid; idx < tg.HB * tg.T * W4; idx += 256) {
      const int hh = (int)(((uint64_t)idx * dinv) >> 20), rem = idx - hh * (int)d;
      const int t = rem / W4, w4 = rem % W4;
      if (hh <= hmax && t < tv)
        *reinterpret_cast<uint4*>(cbase + (uint64_t)(__umul24((uint32_t)hh, NN) + (uint32_t)t) * W + w4 * 4) =
            *reinterpret_cast<const uint4*>(&s_codes[(t * tg.HB + hh) * W + w4 * 4]);
    }
  }
  {
    const uint32_t d = (uint32_t)tg.T * NG, dinv = (1u << 20) / d + 1u;
    uint16_t* sbase = a.scales + ((int64_t)h0 * a.N + i0) * NG;
    for (int idx = tid; idx < tg.HB * tg.T * NG; idx += 256) {
      const int hh = (int)(((uint64_t)idx * dinv) >> 20), rem = idx - hh * (int)d;
      const int t = rem / NG, g = rem % NG;
      if (hh <= hmax && t < tv)
        sbase[(uint64_t)(__umul24((uint32_t)hh, NN) + (uint32_t)t) * NG + g] = s_scales[(t * tg.HB + hh) * NG + g];
    }
  }
}

// Mixed layout (a per-head channel order perm: the 4-bit class first, then the
// 2-bit class, each cut into runs of `group`), same tiles as the uniform
// kernel, in three phases:
//   (1) the residuals of the tile's rows, loaded and formed as in the uniform
//       kernel, into LDS in storage order (channel k at its position in perm,
//       through the inverse order, which starts as the identity so that a perm
//       that is not a permutation still writes inside the row);
//   (2) wave w takes groups w, w + 4, ... of all 64 rows, one row per lane
//       (so the group's width and bits are wave-uniform, and the rows' odd
//       LDS pitch keeps the lanes' reads in distinct banks): it reads the
//       group's residuals as one run, takes the group scale and packs the
//       group's words (groups never share a word: a class starts on a word
//       boundary and `group` is a multiple of 16; positions past a class's
//       end stay zero), into LDS rows ordered (head, token);
//   (3) codes and scales leave per head as contiguous runs.
// Stages that also need the fp32 residual (y_next) take k_quant_pack.
constexpr int kMixMaxWords = 17;     // 4-bit words + 2-bit words of a row (n_int4 = 127)
constexpr int kMixMaxGroups = 9;     // ceil(n_int4 / 16) + ceil((128 - n_int4) / 16)

template <bool F32>
__global__ __launch_bounds__(256) void k_quant_pack_tile_mixed(PackBatch pb, int tiles) {
  __shared__ float s_r[kTileRows][kHeadDim + 5];   // odd pitch: one row per lane in (2)
  __shared__ uint8_t s_inv[kTileHeads][kHeadDim];     // storage position of each channel
  __shared__ uint32_t s_codes[kTileRows * kMixMaxWords];   // rows in (head, token) order
  __shared__ uint16_t s_scales[kTileRows * kMixMaxGroups];
  __shared__ float s_rtab[128];                   // fp32(1 / (1 + k / 128))
  __shared__ int4 s_grp[kMixMaxGroups];           // per group: start, len, bits, first word
  const int tid = threadIdx.x;
  if (tid < 128) s_rtab[tid] = 1.0f / (1.0f + (float)tid * 0.0078125f);
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);   // consecutive tiles share an XCD (L2)
  const PackArgs& a = pb.a[logical / tiles];
  const int tile = (int)(logical % tiles);
  const TileGeom tg = tile_geom(a.H, a.N);
  const int ntb = (a.N + tg.T - 1) / tg.T;
  const int i0 = (tile % ntb) * tg.T, h0 = (tile / ntb) * tg.HB;
  const int tmax = a.N - 1 - i0, hmax = a.H - 1 - h0;
  // row lr of the tile is (token lr / HB, head lr % HB); HB <= 4 and lr < 64, so
  // (lr * hb_inv) >> 16 is the exact quotient
  const uint32_t hb_inv = (65536u + (uint32_t)tg.HB - 1u) / (uint32_t)tg.HB;
  for (int i = tid; i < kTileHeads * kHeadDim; i += 256) s_inv[i >> 7][i & (kHeadDim - 1)] = (uint8_t)(i & (kHeadDim - 1));
  if (tid < a.groups) {
    const GroupInfo gi = group_info(tid, a.bits, a.group, a.n_int4, a.int4_words);
    s_grp[tid] = make_int4(gi.start, gi.len, gi.bits, gi.word0 + gi.pos0 / (32 / gi.bits));
  }
  // (1) residuals; rows outside the tile read a clamped valid row.  Every
  // global load the tile needs is issued before the first barrier -- the
  // heads' perm rows, the labels, the input rows -- then the labelled
  // centroid rows, so the latencies overlap.
  static_assert(kTileHeads * kHeadDim == 2 * 256, "two perm entries per thread");
  const int part = tid & 15, k0 = part * 8;
  constexpr int kIt = kTileRows * 16 / 256;
  const uint32_t ST = (uint32_t)a.y.stride_token, SH = (uint32_t)a.y.stride_head, NN = (uint32_t)a.N;
  const int64_t y_base = (int64_t)i0 * a.y.stride_token + (int64_t)h0 * a.y.stride_head + k0;
  const uint8_t* lab_base = a.labels + (int64_t)h0 * a.N + i0;
  const uint16_t* cent_base = a.centroids + (int64_t)h0 * a.C * kHeadDim + k0;
  uint32_t pv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + 256 * q, hh = i >> 7, p = i & (kHeadDim - 1);
    pv[q] = a.perm[(int64_t)(h0 + min(hh, hmax)) * kHeadDim + p];
  }
  int lab[kIt], hcs[kIt];
  uint32_t yw[kIt][F32 ? 8 : 4];
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    const int lr = x * 16 + (tid >> 4);
    const int t = (int)(((uint32_t)lr * hb_inv) >> 16), hh = lr - t * tg.HB;
    const int tc = min(t, tmax), hc = min(hh, hmax);
    hcs[x] = hc;
    lab[x] = lab_base[__umul24((uint32_t)hc, NN) + (uint32_t)tc];
    const uint32_t yo = __umul24((uint32_t)tc, ST) + __umul24((uint32_t)hc, SH);
    if constexpr (F32) {
      const float* p = reinterpret_cast<const float*>(a.y.ptr) + y_base + yo;
      const uint4 p0 = *reinterpret_cast<const uint4*>(p);
      const uint4 p1 = *reinterpret_cast<const uint4*>(p + 4);
      yw[x][0] = p0.x; yw[x][1] = p0.y; yw[x][2] = p0.z; yw[x][3] = p0.w;
      yw[x][4] = p1.x; yw[x][5] = p1.y; yw[x][6] = p1.z; yw[x][7] = p1.w;
    } else {
      const uint4 p = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.y.ptr) + y_base + yo);
      yw[x][0] = p.x; yw[x][1] = p.y; yw[x][2] = p.z; yw[x][3] = p.w;
    }
  }
  uint4 cw[kIt];
#pragma unroll
  for (int x = 0; x < kIt; ++x)
    cw[x] = *reinterpret_cast<const uint4*>(cent_base + (__umul24((uint32_t)hcs[x], (uint32_t)a.C) +
                                                         (uint32_t)min(lab[x], a.C - 1)) * kHeadDim);
  __syncthreads();                                 // the identity order is in place
  // the first token block of each head block also copies its heads' perm rows
  uint8_t* pout = i0 == 0 ? a.perm_out : nullptr;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + 256 * q, hh = i >> 7, p = i & (kHeadDim - 1);
    s_inv[hh][pv[q] & (kHeadDim - 1)] = (uint8_t)p;
    if (pout && hh <= hmax) pout[(int64_t)(h0 + hh) * kHeadDim + p] = (uint8_t)pv[q];
  }
  __syncthreads();                                 // the storage order is complete
#pragma unroll
  for (int x = 0; x < kIt; ++x) {
    const int lr = x * 16 + (tid >> 4);
    const int hh = lr - (int)(((uint32_t)lr * hb_inv) >> 16) * tg.HB;
    float yv[8], cv[8];
    if constexpr (F32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] = __uint_as_float(yw[x][e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] = bf16_bits_to_f32((yw[x][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
    const uint32_t c4[4] = {cw[x].x, cw[x].y, cw[x].z, cw[x].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) cv[e] = bf16_bits_to_f32((c4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    const uint8_t* inv = s_inv[hh];
#pragma unroll
    for (int e = 0; e < 8; ++e) s_r[lr][inv[k0 + e]] = yv[e] - cv[e];
  }
  __syncthreads();
  // (2) wave w: groups w, w + 4, ... of every row, lane = row
  const int NG = a.groups, W = a.words;
  {
    const int lr = tid & (kTileRows - 1), wave = tid >> 6;
    const int t = (int)(((uint32_t)lr * hb_inv) >> 16), hh = lr - t * tg.HB;
    const int orow = hh * tg.T + t;                // output row: (head, token) order
    const float* rr = s_r[lr];
    // t == T only for lane 63 when HB = 3 (63 rows): not a row of the tile
    for (int g = t < tg.T ? wave : NG; g < NG; g += 4) {
      const int4 gd = s_grp[g];
      const int start = gd.x, len = gd.y, bits = gd.z;
      float amax = 0.0f;
      for (int e0 = 0; e0 < len; e0 += 8) {       // eight reads at a time (past the end: the last again)
        float r8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r8[e] = rr[start + min(e0 + e, len - 1)];
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(r8[e]));
      }
      const float qmax = (float)((1 << (bits - 1)) - 1);
      const uint32_t sbits = f32_to_bf16_bits(amax / qmax);
      const float S = bf16_bits_to_f32(sbits);
      s_scales[orow * NG + g] = (uint16_t)sbits;
      uint32_t* wout = &s_codes[orow * W + gd.w];
      for (int e0 = 0; e0 < len; e0 += 8) {
        float r8[8];
        const int n = min(8, len - e0);
#pragma unroll
        for (int e = 0; e < 8; ++e) r8[e] = e < n ? rr[start + e0 + e] : 0.0f;
        if (bits == 4) {
          uint32_t w = pack8_codes<4>(r8, S, sbits, s_rtab);
          if (n < 8) w &= (1u << (4 * n)) - 1u;
          wout[e0 >> 3] = w;
        } else {
          uint32_t w = pack8_codes<2>(r8, S, sbits, s_rtab);
          if (n < 8) w &= (1u << (2 * n)) - 1u;
          if ((e0 & 8) == 0) wout[e0 >> 4] = w;                 // low half; the high half may follow
          else wout[e0 >> 4] |= w << 16;
        }
      }
    }
  }
  __syncthreads();
  // (3) write-out: per head, the tile's valid rows are one contiguous run of
  // codes and one of scales, in LDS and in the packed layout alike
  const int tv = min(tg.T, a.N - i0);
  for (int hh = 0; hh < tg.HB && hh <= hmax; ++hh) {
    uint32_t* cdst = a.codes + ((int64_t)(h0 + hh) * a.N + i0) * W;
    const uint32_t* csrc = &s_codes[hh * tg.T * W];
    for (int j = tid; j < tv * W; j += 256) cdst[j] = csrc[j];
    uint16_t* sdst = a.scales + ((int64_t)(h0 + hh) * a.N + i0) * NG;
    const uint16_t* ssrc = &s_scales[hh * tg.T * NG];
    for (int j = tid; j < tv * NG; j += 256) sdst[j] = ssrc[j];
  }
}

__device__ __forceinline__ const uint8_t* stage_ptr(const ChunkDecode& d, uint64_t off, uint64_t stride, int l) {
  return d.base + off + stride * (uint64_t)l;
}

// Build the decode table of head h into tab[128] (block-cooperative).  A perm
// that is not a permutation decodes wrongly but stays inside every buffer.
__device__ __forceinline__ void build_table(const ChunkDecode& d, int h, ChannelCode* tab) {
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) tab[p] = ChannelCode{0, 0, (uint8_t)d.bits, 0};
  __syncthreads();
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) {
    const int k = d.n_int4 > 0 ? ((int)(d.base + d.off_perm)[h * kHeadDim + p] & (kHeadDim - 1)) : p;
    tab[k] = code_of(p, d.bits, d.group, d.n_int4, d.int4_words);
  }
}

// x_hat for channels [k0, k0 + n) of token i, head h (fp32 sum over stages in order).
template <int NCH>
__device__ __forceinline__ void dequant_row(const ChunkDecode& d, const ChannelCode* tab, int h, int64_t i,
                                            int k0, float* out) {
#pragma unroll
  for (int e = 0; e < NCH; ++e) out[e] = 0.0f;
  for (int l = 0; l < d.n_stages; ++l) {
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(stage_ptr(d, d.off_codes, d.stage_codes, l)) +
                            ((int64_t)h * d.N + i) * d.words;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(stage_ptr(d, d.off_scales, d.stage_scales, l)) +
                             ((int64_t)h * d.N + i) * d.groups;
    const int lab = min((int)stage_ptr(d, d.off_labels, d.stage_labels, l)[(int64_t)h * d.N + i], d.C - 1);
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(stage_ptr(d, d.off_centroids, d.stage_centroids, l)) +
                           ((int64_t)h * d.C + lab) * kHeadDim;
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const ChannelCode cc = tab[k0 + e];
      const uint32_t u = (codes[cc.word] >> cc.shift) & ((1u << cc.bits) - 1u);
      const float q = (float)((int)u - (1 << (cc.bits - 1)));
      const float S = bf16_bits_to_f32(scales[cc.group]);
      const float yhat = __fadd_rn(S * q, bf16_bits_to_f32(crow[k0 + e]));
      out[e] = l == 0 ? yhat : __fadd_rn(out[e], yhat);
    }
  }
}

// Block: one head, 32 tokens; thread: one token, 16 channels.
__global__ __launch_bounds__(256) void k_dequant(ChunkDecode d, void* out, int out_dtype, int64_t st, int64_t sh) {
  __shared__ ChannelCode tab[kHeadDim];
  const int h = blockIdx.y;
  build_table(d, h, tab);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 32 + threadIdx.x / 8;
  if (i >= d.N) return;
  const int k0 = (threadIdx.x % 8) * 16;
  float v[16];
  dequant_row<16>(d, tab, h, i, k0, v);
  const int64_t o = i * st + (int64_t)h * sh + k0;
  if (out_dtype == 0) {
    float* op = reinterpret_cast<float*>(out) + o;
#pragma unroll
    for (int e = 0; e < 16; ++e) op[e] = v[e];
  } else {
    uint16_t* op = reinterpret_cast<uint16_t*>(out) + o;
#pragma unroll
    for (int e = 0; e < 16; ++e) op[e] = (uint16_t)f32_to_bf16_bits(v[e]);
  }
}

// PSAC encode: e = fp32(x - x_hat) after all stages, coef = bf16(U^T e) from
// float64 dot products.  Block: one head, 256 tokens; thread: one token.
template <bool F32>
__global__ __launch_bounds__(256) void k_psac_encode(ChunkDecode d, TensorView x, const float* __restrict__ U,
                                                     uint16_t* __restrict__ coef) {
  __shared__ ChannelCode tab[kHeadDim];
  __shared__ float sU[kHeadDim * kMaxRank];
  const int h = blockIdx.y;
  const int r = d.psac_rank;
  build_table(d, h, tab);
  for (int idx = threadIdx.x; idx < kHeadDim * r; idx += blockDim.x) sU[idx] = U[(int64_t)h * kHeadDim * r + idx];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= d.N) return;
  double acc[kMaxRank];
#pragma unroll
  for (int b = 0; b < kMaxRank; ++b) acc[b] = 0.0;
  for (int k0 = 0; k0 < kHeadDim; k0 += 16) {
    float v[16];
    dequant_row<16>(d, tab, h, i, k0, v);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float err = __fsub_rn(load_y<F32>(x, i, h, k0 + e), v[e]);
#pragma unroll
      for (int b = 0; b < kMaxRank; ++b)
        if (b < r) acc[b] += (double)sU[(k0 + e) * r + b] * (double)err;
    }
  }
  uint16_t* cp = coef + ((int64_t)h * d.N + i) * r;
#pragma unroll
  for (int b = 0; b < kMaxRank; ++b)
    if (b < r) cp[b] = (uint16_t)f64_to_bf16_bits(acc[b]);
}

}  // namespace

hipError_t launch_quant_pack_generic(const PackArgs& a, hipStream_t s) {
  TimedLaunch tl_("k_quant_pack", s);
  const bool f32 = a.y.dtype == 0;
  const int64_t total = (int64_t)a.H * a.N * a.groups;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define QKV_QP(GV)                                                              \
  if (a.group == GV) {                                                          \
    if (f32) hipLaunchKernelGGL((k_quant_pack<GV, true>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((k_quant_pack<GV, false>), grid, block, 0, s, a);    \
    return hipGetLastError();                                                   \
  }
  QKV_QP(16)
  QKV_QP(32)
  QKV_QP(64)
  QKV_QP(128)
#undef QKV_QP
  return hipErrorInvalidValue;
}

hipError_t launch_quant_pack(const PackArgs& a, hipStream_t s) {
  if (!a.perm && a.n_int4 == 0) {
    PackBatch pb;
    pb.n = 1;
    pb.a[0] = a;
    return launch_quant_pack_batch(pb, s);
  }
  if (quant_pack_mixed_batchable(a, a)) {
    PackBatch pb;
    pb.n = 1;
    pb.a[0] = a;
    return launch_quant_pack_mixed_batch(pb, s);
  }
  if (a.perm && a.perm_out) {
    const hipError_t e = launch_copy_perm(a.perm, a.perm_out, a.H, s);
    if (e != hipSuccess) return e;
  }
  return launch_quant_pack_generic(a, s);
}

// the mixed tile kernel: no fp32 residual output, 24-bit in-tile offsets
bool quant_pack_mixed_batchable(const PackArgs& a, const PackArgs& b0) {
  const bool tile_ok = a.perm && !a.y_next && a.words <= kMixMaxWords && a.groups <= kMixMaxGroups &&
                       a.y.stride_token < (1 << 23) && a.y.stride_head < (1 << 23) && a.N < (1 << 23) &&
                       (int64_t)a.H * a.C < (1 << 23);
  return tile_ok && b0.perm && !b0.y_next && a.y.dtype == b0.y.dtype && a.H == b0.H && a.N == b0.N &&
         a.C == b0.C && a.bits == b0.bits && a.group == b0.group && a.n_int4 == b0.n_int4 &&
         a.int4_words == b0.int4_words && a.words == b0.words && a.groups == b0.groups;
}

hipError_t launch_quant_pack_mixed_batch(const PackBatch& b, hipStream_t s) {
  const PackArgs& a = b.a[0];
  for (int p = 0; p < b.n; ++p)
    if (!quant_pack_mixed_batchable(b.a[p], a)) return hipErrorInvalidValue;
  TimedLaunch tl_("k_quant_pack_tile_mixed", s);
  const int tiles = tile_geom(a.H, a.N).tiles;
  const dim3 grid((unsigned)(tiles * b.n)), block(256);
  if (a.y.dtype == 0) hipLaunchKernelGGL(k_quant_pack_tile_mixed<true>, grid, block, 0, s, b, tiles);
  else hipLaunchKernelGGL(k_quant_pack_tile_mixed<false>, grid, block, 0, s, b, tiles);
  return hipGetLastError();
}

bool quant_pack_batchable(const PackArgs& a, const PackArgs& b0) {
  return !a.perm && a.n_int4 == 0 && a.group == b0.group && a.bits == b0.bits && a.y.dtype == b0.y.dtype &&
         a.H == b0.H && a.N == b0.N;
}

hipError_t launch_quant_pack_batch(const PackBatch& b, hipStream_t s) {
  const PackArgs& a = b.a[0];
  for (int p = 0; p < b.n; ++p)
    if (!quant_pack_batchable(b.a[p], a)) return hipErrorInvalidValue;
  if (a.words != kHeadDim * a.bits / 32 || a.groups != kHeadDim / a.group) return hipErrorInvalidValue;
  // the tile kernel forms in-tile offsets with 24-bit multiplies
  bool small = true;
  for (int p = 0; p < b.n; ++p)
    small = small && b.a[p].y.stride_token < (1 << 23) && b.a[p].y.stride_head < (1 << 23) && b.a[p].N < (1 << 23);
  if (!small) {
    for (int p = 0; p < b.n; ++p) {
      hipError_t e = launch_quant_pack_generic(b.a[p], s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const bool f32 = a.y.dtype == 0;
  const int tiles = tile_geom(a.H, a.N).tiles;
  const dim3 grid((unsigned)(tiles * b.n)), block(256);
  TimedLaunch tl_("k_quant_pack_tile", s);
#define QKV_QF(GV, BV)                                                                              \
  if (a.group == GV && a.bits == BV) {                                                              \
    if (f32) hipLaunchKernelGGL((k_quant_pack_tile<GV, BV, true>), grid, block, 0, s, b, tiles);     \
    else hipLaunchKernelGGL((k_quant_pack_tile<GV, BV, false>), grid, block, 0, s, b, tiles);        \
    return hipGetLastError();                                                                       \
  }
  QKV_QF(16, 2) QKV_QF(32, 2) QKV_QF(64, 2) QKV_QF(128, 2)
  QKV_QF(16, 4) QKV_QF(32, 4) QKV_QF(64, 4) QKV_QF(128, 4)
#undef QKV_QF
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize(const ChunkDecode& d, void* out, int out_dtype, int64_t stride_token,
                             int64_t stride_head, hipStream_t s) {
  TimedLaunch tl_("k_dequant", s);
  const dim3 grid((unsigned)((d.N + 31) / 32), (unsigned)d.H);
  hipLaunchKernelGGL(k_dequant, grid, dim3(256), 0, s, d, out, out_dtype, stride_token, stride_head);
  return hipGetLastError();
}

hipError_t launch_psac_encode(const ChunkDecode& d, const TensorView& x, const float* U, uint16_t* coef_out,
                              hipStream_t s) {
  TimedLaunch tl_("k_psac_encode", s);
  const dim3 grid((unsigned)((d.N + 255) / 256), (unsigned)d.H);
  if (x.dtype == 0) hipLaunchKernelGGL(k_psac_encode<true>, grid, dim3(256), 0, s, d, x, U, coef_out);
  else hipLaunchKernelGGL(k_psac_encode<false>, grid, dim3(256), 0, s, d, x, U, coef_out);
  return hipGetLastError();
}

hipError_t launch_copy_perm(const uint8_t* perm, uint8_t* dst, int H, hipStream_t s) {
  TimedLaunch tl_("copy_perm", s);
  return hipMemcpyAsync(dst, perm, (size_t)H * kHeadDim, hipMemcpyDeviceToDevice, s);
}

}  // namespace qkv
