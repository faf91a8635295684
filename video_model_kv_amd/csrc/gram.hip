// Second-moment matrix of the history queries per head, M_h = sum_n q_n q_n^T,
// in float64 (QuantWM summary, "QuantWM": QSAC reads the per-channel activity
// diag(M)/n, PSAC eigendecomposes M).  This is a cold path (once per history
// window), so it favours exactness over speed: products of bf16 queries are
// exact in float64 and every partial sum is accumulated in a fixed order.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

constexpr int kRows = 32;

// Block (split, head): rows [split * rows_per, ...).  Thread t owns row a = t/2
// and columns [64 * (t%2), +64) of M.
template <bool F32>
__global__ __launch_bounds__(256) void k_gram_partial(TensorView q, int n_split, double* __restrict__ partial) {
  __shared__ double sq[kRows][kHeadDim];
  const int split = blockIdx.x, h = blockIdx.y, H = gridDim.y;
  const int64_t n = q.n_tokens;
  const int64_t rows_per = (n + n_split - 1) / n_split;
  const int64_t r0 = split * rows_per, r1 = min(n, r0 + rows_per);
  const int a = threadIdx.x >> 1, b0 = (threadIdx.x & 1) * 64;
  double acc[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) acc[c] = 0.0;
  for (int64_t base = r0; base < r1; base += kRows) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kRows * kHeadDim; idx += 256) {
      const int rr = idx / kHeadDim, k = idx % kHeadDim;
      const int64_t row = base + rr;
      double v = 0.0;
      if (row < r1) {
        const int64_t off = row * q.stride_token + (int64_t)h * q.stride_head + k;
        if constexpr (F32) v = (double)reinterpret_cast<const float*>(q.ptr)[off];
        else v = (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q.ptr)[off]);
      }
      sq[rr][k] = v;
    }
    __syncthreads();
    for (int rr = 0; rr < kRows; ++rr) {
      const double qa = sq[rr][a];
#pragma unroll
      for (int c = 0; c < 64; ++c) acc[c] += qa * sq[rr][b0 + c];
    }
  }
  double* out = partial + (((int64_t)split * H + h) * kHeadDim + a) * kHeadDim + b0;
#pragma unroll
  for (int c = 0; c < 64; ++c) out[c] = acc[c];
}

__global__ void k_gram_reduce(int64_t per, int n_split, const double* __restrict__ partial, double* __restrict__ m) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per) return;
  double s = 0.0;
  for (int k = 0; k < n_split; ++k) s += partial[(int64_t)k * per + i];
  m[i] = s;
}

}  // namespace

hipError_t launch_gram(const TensorView& q, int H, double* partial, int n_split, double* m, hipStream_t s) {
  TimedLaunch tl_("k_gram", s);
  const dim3 grid(n_split, H);
  if (q.dtype == 0) hipLaunchKernelGGL(k_gram_partial<true>, grid, dim3(256), 0, s, q, n_split, partial);
  else hipLaunchKernelGGL(k_gram_partial<false>, grid, dim3(256), 0, s, q, n_split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per = (int64_t)H * kHeadDim * kHeadDim;
  hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, s, per, n_split, partial, m);
  return hipGetLastError();
}

}  // namespace qkv
