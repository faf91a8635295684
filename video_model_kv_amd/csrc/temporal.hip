// Temporally stable 2-bit KV codec (practitioner blog, sections 3.3-3.5):
// outlier separation at the block's P99 into fp16, asymmetric min/max codes
// with a per-block fp16 zero point and scale, fp16 anchor frames every
// `anchor_every` frames with the other frames coded as their delta to the
// anchor, and error feedback (the error of frame t against the uncompensated
// values, times `decay`, added to frame t + 1 before it is coded).
//
// Readings (the page is silent, or its pseudo-code lost its operators):
//   - a block is one token-head's run of 32 consecutive channels;
//   - P99 by linear interpolation over a 32-value block lies strictly between
//     the two largest magnitudes when they differ: the outlier is the block's
//     largest magnitude when unique (lowest channel), none otherwise;
//   - lo = fp16(min), S = fp16((max - lo) / (2^b - 1)) over the non-outliers,
//     q = clamp(rint((r - lo) / S), 0, 2^b - 1) (S <= 0: q = 0), rebuilt as
//     lo + q S; the outlier rebuilds as its fp16 value;
//   - the prediction of a frame is its group's anchor as stored, position by
//     position; anchor frames store fp16(kv) uncompensated;
//   - every operation is one float32 rounding in the order written, fp16
//     conversions round to nearest even.
//
// Layout of the work: the chunk's frames are serial (the feedback loop), the
// (position, head, block) triples are independent.  Each lane takes 4
// consecutive channels through all frames of the call, their feedback and
// anchor in registers; eight lanes form a block, whose statistics are three
// DPP exchanges each (no LDS).
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

__device__ __forceinline__ float to_f16f(float x) { return (float)(_Float16)x; }   // nearest even

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Exchanges inside a group of 8 lanes (DPP, all lanes active): swap neighbours,
// swap pairs, then mirror the two quads.  After the three steps of a reduction
// every lane of the group holds the group's result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t g8_reduce(uint32_t v, Op op) {
  v = op(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4E>(v));     // quad_perm [2,3,0,1]
  v = op(v, dpp<0x141>(v));    // row half mirror
  return v;
}
__device__ __forceinline__ float g8_max(float v) {
  return __uint_as_float(g8_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float g8_min(float v) {
  return __uint_as_float(g8_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float g8_sum(float v) {   // exact here: at most one nonzero term
  return __uint_as_float(g8_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ uint32_t g8_add_u(uint32_t v) {
  return g8_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t g8_min_u(uint32_t v) {
  return g8_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Lane l of wave gw holds channels 4 (l % 32) .. + 3 of token-head 2 gw + l / 32;
// eight lanes form a 32-channel block.
template <bool F32>
__global__ __launch_bounds__(256) void k_tenc(TCodecArgs a) {
  const int lane = threadIdx.x & 63;
  const uint32_t n_th = (uint32_t)a.P * (uint32_t)a.H;
  const uint32_t gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw * 2 >= n_th) return;                                         // whole waves only
  const uint32_t th = min(gw * 2 + (lane >> 5), n_th - 1);            // token-head = position * H + head
  const bool live = gw * 2 + (lane >> 5) < n_th;                      // the odd last token-head: a copy, not stored
  const int p = (int)(th / (uint32_t)a.H), h = (int)(th % (uint32_t)a.H);
  const int c0 = 4 * (lane & 31);                                     // first channel of the lane
  const int blk = c0 >> 5, g8 = lane & 7;                             // block; lane within the block
  const int64_t e = (int64_t)th * kHeadDim + c0;                      // element of a frame / the state
  float fb[4], anc[4];
  {
    const float4 f4 = *reinterpret_cast<const float4*>(a.fb + e);
    fb[0] = f4.x; fb[1] = f4.y; fb[2] = f4.z; fb[3] = f4.w;
    const uint2 a2 = *reinterpret_cast<const uint2*>(a.anchor + e);
    anc[0] = f16_bits_to_f32(a2.x & 0xFFFFu); anc[1] = f16_bits_to_f32(a2.x >> 16);
    anc[2] = f16_bits_to_f32(a2.y & 0xFFFFu); anc[3] = f16_bits_to_f32(a2.y >> 16);
  }
  const float levels = (float)((1 << a.bits) - 1);
  for (int f = 0; f < a.n_frames; ++f) {
    const int64_t off = ((int64_t)f * a.P + p) * a.x.stride_token + (int64_t)h * a.x.stride_head + c0;
    float x[4];
    if constexpr (F32) {
      const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x.ptr) + off);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x.ptr) + off);
      x[0] = bf16_bits_to_f32(v.x & 0xFFFFu); x[1] = bf16_bits_to_f32(v.x >> 16);
      x[2] = bf16_bits_to_f32(v.y & 0xFFFFu); x[3] = bf16_bits_to_f32(v.y >> 16);
    }
    uint8_t* fr = a.packed + a.frame_off[f];
    float kv_hat[4];
    if ((a.frame0 + f) % a.anchor_every == 0) {
      uint16_t b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        b[k] = f16_bits(x[k]);
        anc[k] = f16_bits_to_f32(b[k]);
        kv_hat[k] = anc[k];
      }
      if (live)
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(fr) + e) =
            make_uint2(b[0] | ((uint32_t)b[1] << 16), b[2] | ((uint32_t)b[3] << 16));
    } else {
      float r[4], mag[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float comp = x[k] + fb[k];
        r[k] = comp - anc[k];
        mag[k] = fabsf(r[k]);
      }
      const float top = g8_max(fmaxf(fmaxf(mag[0], mag[1]), fmaxf(mag[2], mag[3])));
      uint32_t cnt = 0, first = 255;
      float rtop = 0.0f;
#pragma unroll
      for (int k = 3; k >= 0; --k)
        if (mag[k] == top) {
          ++cnt;
          first = (uint32_t)(4 * g8 + k);
          rtop = r[k];
        }
      const bool unique = g8_add_u(cnt) == 1;
      const uint32_t fidx = g8_min_u(first);                          // lowest channel at the top
      const float r_out = g8_sum(unique && first == fidx ? rtop : 0.0f);
      bool out[4];
      float lmn = INFINITY, lmx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[k] = unique && (uint32_t)(4 * g8 + k) == fidx;
        lmn = fminf(lmn, out[k] ? INFINITY : r[k]);
        lmx = fmaxf(lmx, out[k] ? -INFINITY : r[k]);
      }
      const float lo = to_f16f(g8_min(lmn));
      const float S = to_f16f((g8_max(lmx) - lo) / levels);
      uint32_t qb = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float q = 0.0f;
        if (S > 0.0f && !out[k]) q = fminf(fmaxf(__builtin_rintf((r[k] - lo) / S), 0.0f), levels);
        const float r_hat = out[k] ? to_f16f(r[k]) : lo + q * S;
        kv_hat[k] = anc[k] + r_hat;
        qb |= (uint32_t)q << (a.bits * k);
      }
      // codes: a word holds 32 / bits channels = 8 / bits lanes
      uint32_t* codes = reinterpret_cast<uint32_t*>(fr + a.sec_codes);
      if (a.bits == 2) {
        uint32_t w = qb << (8 * (lane & 3));
        w |= dpp<0xB1>(w);
        w |= dpp<0x4E>(w);
        if (live && (lane & 3) == 0) codes[(int64_t)th * 8 + blk * 2 + (g8 >> 2)] = w;
      } else {
        uint32_t w = qb << (16 * (lane & 1));
        w |= dpp<0xB1>(w);
        if (live && (lane & 1) == 0) codes[(int64_t)th * 16 + blk * 4 + (g8 >> 1)] = w;
      }
      if (live && g8 == 0) {
        const int64_t bi = (int64_t)th * 4 + blk;
        reinterpret_cast<uint16_t*>(fr + a.sec_lo)[bi] = f16_bits(lo);
        reinterpret_cast<uint16_t*>(fr + a.sec_scale)[bi] = f16_bits(S);
        reinterpret_cast<uint16_t*>(fr + a.sec_oval)[bi] = unique ? f16_bits(r_out) : 0;
        (fr + a.sec_oidx)[bi] = unique ? (uint8_t)fidx : (uint8_t)255;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) fb[k] = a.decay * (x[k] - kv_hat[k]);
  }
  if (live) {
    *reinterpret_cast<float4*>(a.fb + e) = make_float4(fb[0], fb[1], fb[2], fb[3]);
    uint16_t b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) b[k] = f16_bits(anc[k]);
    *reinterpret_cast<uint2*>(a.anchor + e) = make_uint2(b[0] | ((uint32_t)b[1] << 16), b[2] | ((uint32_t)b[3] << 16));
  }
}

// One thread per 4 channels of a token-head, all frames of the run in order
// (anc_frame[f]: the run's frame holding frame f's anchor, -1 = the caller's).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_tdec(TCodecArgs a, void* out, int64_t out_st, int64_t out_sh) {
  const uint32_t n_th = (uint32_t)a.P * (uint32_t)a.H;
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_th * 32) return;
  const uint32_t th = i >> 5;
  const int c0 = 4 * (int)(i & 31), blk = c0 >> 5, g8 = (c0 & 31) >> 2;
  const int p = (int)(th / (uint32_t)a.H), h = (int)(th % (uint32_t)a.H);
  const int64_t e = (int64_t)th * kHeadDim + c0;
  float anc[4];
  int cur = -2;                                       // which anchor anc holds
  const int per = 32 / a.bits;
  for (int f = 0; f < a.n_frames; ++f) {
    const int fa = a.anc_frame[f];
    if (fa != cur) {
      const uint16_t* src = fa >= 0 ? reinterpret_cast<const uint16_t*>(a.packed + a.frame_off[fa]) : a.anchor;
      const uint2 v = *reinterpret_cast<const uint2*>(src + e);
      anc[0] = f16_bits_to_f32(v.x & 0xFFFFu); anc[1] = f16_bits_to_f32(v.x >> 16);
      anc[2] = f16_bits_to_f32(v.y & 0xFFFFu); anc[3] = f16_bits_to_f32(v.y >> 16);
      cur = fa;
    }
    float kv_hat[4];
    if (fa == f) {
#pragma unroll
      for (int k = 0; k < 4; ++k) kv_hat[k] = anc[k];
    } else {
      const uint8_t* fr = a.packed + a.frame_off[f];
      const int wi = (c0 & 31) / per;
      const uint32_t w = reinterpret_cast<const uint32_t*>(fr + a.sec_codes)[(int64_t)th * (4 * a.bits) + blk * a.bits + wi];
      const uint32_t qb = w >> (a.bits * ((c0 & 31) % per));
      const int64_t bi = (int64_t)th * 4 + blk;
      const float lo = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(fr + a.sec_lo)[bi]);
      const float S = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(fr + a.sec_scale)[bi]);
      const int oi = (fr + a.sec_oidx)[bi];
      const float ov = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(fr + a.sec_oval)[bi]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float q = (float)((qb >> (a.bits * k)) & ((1u << a.bits) - 1));
        const float r_hat = oi == 4 * g8 + k ? ov : lo + q * S;
        kv_hat[k] = anc[k] + r_hat;
      }
    }
    const int64_t o = ((int64_t)f * a.P + p) * out_st + (int64_t)h * out_sh + c0;
    if constexpr (OUT_BF16) {
      uint32_t b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = f32_to_bf16_bits(kv_hat[k]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o) = make_float4(kv_hat[0], kv_hat[1], kv_hat[2], kv_hat[3]);
    }
  }
}

}  // namespace

hipError_t launch_temporal_encode(const TCodecArgs& a, hipStream_t s) {
  TimedLaunch tl_("k_tenc", s);
  const int64_t waves = ((int64_t)a.P * a.H + 1) / 2;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (a.x.dtype == 0) hipLaunchKernelGGL(k_tenc<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_tenc<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_temporal_decode(const TCodecArgs& a, void* out, int out_dtype, int64_t out_st, int64_t out_sh,
                                  hipStream_t s) {
  TimedLaunch tl_("k_tdec", s);
  const int64_t n = (int64_t)a.P * a.H * 32;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (out_dtype == 0) hipLaunchKernelGGL(k_tdec<false>, grid, dim3(256), 0, s, a, out, out_st, out_sh);
  else hipLaunchKernelGGL(k_tdec<true>, grid, dim3(256), 0, s, a, out, out_st, out_sh);
  return hipGetLastError();
}

}  // namespace qkv
