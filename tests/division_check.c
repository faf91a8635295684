/*
 * CPU brute force of the quotient shortcut in the tiled quant-pack kernel
 * (test infrastructure; compiled and run by tests/test_division_check.py).
 *
 * The kernel forms q = rint(fp32(r / S)) for a bf16 scale S with 2^-96 <= S <
 * 2^96 without a division: rS = fp32(1 / m) * 2^-e from a 128-entry table over
 * the bf16 significands m = 1 + k/128, x0 = fp32(r * rS), then one refinement
 * x = fma(fma(-x0, S, r), rS, x0), and finally rint with ties to even.  This
 * program draws residuals of several kinds (exact and near half-integer
 * quotients, random ones, bf16-valued ones, full-significand ones) and counts
 * the samples where rint(x) differs from rint of the correctly rounded
 * quotient, and where x differs from fp32(r / S) at all.
 * Usage: division_check <samples>; exit status 1 on any code mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static float as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t as_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float to_bf16(float f) {                 /* round to nearest even */
  uint32_t u = as_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return as_float(u & 0xFFFF0000u);
}
static float uniform(void) { return (float)((double)(next() % 2000001) / 1000000.0 - 1.0); }

int main(int argc, char** argv) {
  const long samples = argc > 1 ? atol(argv[1]) : 1000000;
  float table[128];
  for (int k = 0; k < 128; ++k) table[k] = 1.0f / (1.0f + (float)k / 128.0f);
  long code_mismatch = 0, quotient_differs = 0, exact_half = 0;
  for (long i = 0; i < samples; ++i) {
    const int qmax = (next() & 1) ? 1 : 7;
    const float S = to_bf16(ldexpf(1.0f + (float)(next() % 128) / 128.0f, (int)(next() % 181) - 90));
    float r;
    const int kind = (int)(next() % 5);
    if (kind == 0 || kind == 1) {                /* on, or up to 4 ulp from, a half-integer quotient */
      const float half = (float)((int)(next() % (2 * qmax)) - qmax) + 0.5f;
      r = half * S;                              /* exact: at most 12 significant bits */
      const int nudge = (int)(next() % 9) - 4;
      if (nudge == 0) ++exact_half;
      r = as_float(as_bits(r) + (uint32_t)nudge);
      if (kind == 1) r = -r;
    } else if (kind == 2) {
      r = uniform() * (float)qmax * S;
    } else if (kind == 3) {
      r = to_bf16(uniform() * (float)qmax * S);
    } else {
      const uint32_t m = (uint32_t)(next() & 0x7FFFFF);
      r = ldexpf(as_float(0x3F800000u | m), (int)(next() % 4) - 3) * S * ((next() & 1) ? 1.0f : -1.0f) *
          (float)qmax * 0.999f;
    }
    const float exact = r / S;                   /* correctly rounded (IEEE division) */
    const uint32_t sb = as_bits(S) >> 16;        /* bf16 bits of S */
    const int E = (int)((sb >> 7) & 0xFF);
    const float rS = ldexpf(table[sb & 0x7F], 127 - E);
    float x = r * rS;
    x = fmaf(fmaf(-x, S, r), rS, x);
    if (as_bits(x) != as_bits(exact)) ++quotient_differs;
    if (rintf(x) != rintf(exact)) ++code_mismatch;
  }
  printf("samples %ld exact-half-integer %ld quotient-differs %ld code-mismatch %ld\n", samples, exact_half,
         quotient_differs, code_mismatch);
  return code_mismatch != 0 || quotient_differs != 0;
}
