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

// The diagonal alone (QSAC's activity and the mixed layout's channel order
// need no more): block (split, head), thread = channel, the split's rows in
// the same order as k_gram_partial, so every value is the same as that
// kernel's diagonal.
template <bool F32>
__global__ __launch_bounds__(kHeadDim) void k_gram_diag_partial(TensorView q, int n_split, double* __restrict__ partial) {
  const int split = blockIdx.x, h = blockIdx.y, H = gridDim.y, k = threadIdx.x;
  const int64_t n = q.n_tokens;
  const int64_t rows_per = (n + n_split - 1) / n_split;
  const int64_t r0 = split * rows_per, r1 = min(n, r0 + rows_per);
  const int64_t off0 = (int64_t)h * q.stride_head + k;
  double acc = 0.0;
#pragma unroll 8
  for (int64_t row = r0; row < r1; ++row) {
    double v;
    if constexpr (F32) v = (double)reinterpret_cast<const float*>(q.ptr)[row * q.stride_token + off0];
    else v = (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q.ptr)[row * q.stride_token + off0]);
    acc += v * v;
  }
  partial[((int64_t)split * H + h) * kHeadDim + k] = acc;
}

__global__ void k_gram_reduce(int64_t per, int n_split, const double* __restrict__ partial, double* __restrict__ m) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per) return;
  double s = 0.0;
  for (int k = 0; k < n_split; ++k) s += partial[(int64_t)k * per + i];
  m[i] = s;
}

// QSAC's second factor (QuantWM summary, "QuantWM", first technique: the
// clustering also weighs the dynamic range of the residual being quantized).
// Block (head, split) of problem blockIdx.y: each lane keeps the running minimum
// and maximum of two channels over the split's tokens (waves stride by 4
// tokens); the four waves are joined in LDS.  Minima and maxima are exact, so
// the split order is immaterial.
template <bool F32>
__global__ __launch_bounds__(256) void k_range_partial(RangeBatch b) {
  const int p = blockIdx.y;
  const int h = blockIdx.x / kRangeSplits, sp = blockIdx.x % kRangeSplits;
  const int64_t t0 = b.N * sp / kRangeSplits, t1 = b.N * (sp + 1) / kRangeSplits;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
  const int64_t hoff = (int64_t)h * b.stride_head[p] + lane * 2;
#pragma unroll 4
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    const int64_t off = t * b.stride_token[p] + hoff;
    float a, c;
    if constexpr (F32) {
      const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(b.y[p]) + off);
      a = v.x;
      c = v.y;
    } else {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(b.y[p]) + off);
      a = bf16_bits_to_f32(v & 0xFFFFu);
      c = bf16_bits_to_f32(v >> 16);
    }
    mn0 = fminf(mn0, a);
    mx0 = fmaxf(mx0, a);
    mn1 = fminf(mn1, c);
    mx1 = fmaxf(mx1, c);
  }
  __shared__ float sm[4][4][64];
  sm[wave][0][lane] = mn0;
  sm[wave][1][lane] = mn1;
  sm[wave][2][lane] = mx0;
  sm[wave][3][lane] = mx1;
  __syncthreads();
  if (wave == 0) {
    for (int x = 1; x < 4; ++x) {
      mn0 = fminf(mn0, sm[x][0][lane]);
      mn1 = fminf(mn1, sm[x][1][lane]);
      mx0 = fmaxf(mx0, sm[x][2][lane]);
      mx1 = fmaxf(mx1, sm[x][3][lane]);
    }
    float* out = b.part[p] + ((int64_t)h * kRangeSplits + sp) * 2 * kHeadDim;
    *reinterpret_cast<float2*>(out + lane * 2) = make_float2(mn0, mn1);
    *reinterpret_cast<float2*>(out + kHeadDim + lane * 2) = make_float2(mx0, mx1);
  }
}

// Block (head) of problem blockIdx.y, thread = channel: the range over the
// splits and the combined weight, each float operation rounded once.
__global__ __launch_bounds__(kHeadDim) void k_range_weights(RangeBatch b) {
  const int p = blockIdx.y, h = blockIdx.x, k = threadIdx.x;
  const float* part = b.part[p] + (int64_t)h * kRangeSplits * 2 * kHeadDim;
  float mn = INFINITY, mx = -INFINITY;
  for (int sp = 0; sp < kRangeSplits; ++sp) {
    mn = fminf(mn, part[sp * 2 * kHeadDim + k]);
    mx = fmaxf(mx, part[sp * 2 * kHeadDim + kHeadDim + k]);
  }
  const float rho = mx - mn;
  const float rr = rho * rho;
  b.w_out[p][h * kHeadDim + k] = b.wq[p][h * kHeadDim + k] * rr;
}

}  // namespace

hipError_t launch_qsac_range(const RangeBatch& b, hipStream_t s) {
  if (b.n <= 0) return hipSuccess;
  {
    TimedLaunch tl_("k_range_partial", s);
    const dim3 grid((unsigned)(b.H * kRangeSplits), (unsigned)b.n);
    if (b.dtype == 0) hipLaunchKernelGGL(k_range_partial<true>, grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL(k_range_partial<false>, grid, dim3(256), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TimedLaunch tl_("k_range_weights", s);
  hipLaunchKernelGGL(k_range_weights, dim3((unsigned)b.H, (unsigned)b.n), dim3(kHeadDim), 0, s, b);
  return hipGetLastError();
}

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

hipError_t launch_gram_diag(const TensorView& q, int H, double* partial, int n_split, double* m, hipStream_t s) {
  TimedLaunch tl_("k_gram_diag", s);
  const dim3 grid(n_split, H);
  if (q.dtype == 0) hipLaunchKernelGGL(k_gram_diag_partial<true>, grid, dim3(kHeadDim), 0, s, q, n_split, partial);
  else hipLaunchKernelGGL(k_gram_diag_partial<false>, grid, dim3(kHeadDim), 0, s, q, n_split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per = (int64_t)H * kHeadDim;
  hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, s, per, n_split, partial, m);
  return hipGetLastError();
}

}  // namespace qkv
