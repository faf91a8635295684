// Device-side helpers shared by the libqkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace qkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  // round to nearest even by the hardware conversion (v_cvt_pk_bf16_f32 on
  // gfx950; fp32 subnormals are kept): for every finite f the same bits as
  // adding 0x7FFF + the lowest kept bit and truncating
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// double -> bfloat16 bits with a single round-to-nearest-even (normal range;
// results below the bf16 normal range go through float, which is adequate for
// magnitudes under 2^-126).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  if (x == 0.0) return (uint32_t)(__double_as_longlong(x) >> 48) & 0x8000u;
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(u >> 63);
  int e = (int)((u >> 52) & 0x7FF) - 1023;
  if (e < -126) return f32_to_bf16_bits((float)x);
  uint64_t v = ((uint64_t)(e + 127) << 52) | (u & ((1ull << 52) - 1));
  v = (v + (1ull << 44) - 1 + ((v >> 45) & 1ull)) >> 45;   // 8-bit exponent, 7-bit fraction
  if (v >= 0x7F80u) v = 0x7F80u;                           // overflow -> infinity
  return (sign << 15) | (uint32_t)v;
}

// Error-free transformation: s + e == a + b exactly.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Double-double accumulator (hi, lo): hi is always the float64 rounding of hi + lo.
struct DD {
  double hi, lo;
  __device__ __forceinline__ void add(double x) {
    double s, e;
    two_sum(hi, x, s, e);
    e += lo;
    hi = s + e;
    lo = e - (hi - s);
  }
  __device__ __forceinline__ void add(const DD& o) {
    double s, e;
    two_sum(hi, o.hi, s, e);
    e += lo + o.lo;
    hi = s + e;
    lo = e - (hi - s);
  }
};

// Block index remapping so that consecutive logical blocks land on the same
// XCD (the dispatcher deals workgroups to the 8 XCDs round-robin).  Bijective
// on [0, total).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t linear, uint32_t total) {
  const uint32_t nx = 8;
  uint32_t x = linear % nx, slot = linear / nx;
  uint32_t per = total / nx, rem = total % nx;
  uint32_t base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + slot;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait for vmcnt <= n only, or for lgkmcnt == 0 only
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;

// Asynchronous global -> LDS copy of 16 bytes per lane: lane i's bytes land at
// dst + 16 i (dst wave-uniform).  Tracked by vmcnt; a workgroup barrier after
// the wait makes them visible to the other waves.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_ptr)const_cast<void*>(src), (lds_ptr)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {   // 4 bytes per lane at dst + 4 i
  __builtin_amdgcn_global_load_lds((glb_ptr)const_cast<void*>(src), (lds_ptr)dst, 4, 0, 0);
}

}  // namespace qkv
