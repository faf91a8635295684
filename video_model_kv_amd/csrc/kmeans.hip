// k-means of one chunk's tokens per head: strided init, MFMA distance GEMM with
// wave argmin (assign), exact-sum centroid means (update).
//
// Method: Quant VideoGen notes, "Key designs / Semantic-Aware Smoothing" (the
// chunk's tokens are grouped by k-means and each group gets its mean as a
// centroid); QuantWM summary, "QuantWM", first technique (QSAC: per-channel
// query-activity weights w in the distance).
//
// Assign computes, for every token y and centroid c,
//     D'(y, c) = sum_k w_k c_k^2 - 2 sum_k y_k (w_k c_k)
// which differs from the weighted squared distance by sum_k w_k y_k^2, a
// per-token constant that does not move the argmin.  The dot products run on
// MFMA (v_mfma_f32_32x32x16_bf16): fp32(w*c) is split into bf16 hi + lo (16
// significant bits), bf16 tokens are exact operands, fp32 tokens are split
// into hi + lo too (three products: hh, lh, hl); products are exact and the
// sums are fp32.  The error of D' stays below ~1e-6 of ||y||_w^2 + ||c||_w^2;
// every token whose two best screened values are closer than 2e-5 of that
// scale is re-decided from float64 distances accumulated in channel order, so
// the labels are those of the float64 definition (ties to the lowest index).
#include "common.h"
#include "kernels.h"

namespace qkv {

namespace {

constexpr int kAssignTokens = 256;   // 4 waves x 64 tokens
constexpr int kPitch = 136;          // LDS row pitch (bf16): 128 + 8 keeps ds_read_b128 conflict-free

template <bool F32>
__device__ __forceinline__ float load1(const TensorView& y, int64_t tok, int h, int k) {
  const int64_t off = tok * y.stride_token + (int64_t)h * y.stride_head + k;
  if constexpr (F32) return reinterpret_cast<const float*>(y.ptr)[off];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(y.ptr)[off]);
}

// Block (head, 8 centroids): c_j = y[j * floor(N / C)] as float32.
template <bool F32>
__global__ __launch_bounds__(256) void k_init(TensorView y, int C, float* __restrict__ c) {
  const int h = blockIdx.y;
  const int j = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (j >= C) return;
  const int64_t step = y.n_tokens / C;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = (threadIdx.x & 31) * 4 + e;
    c[((int64_t)h * C + j) * kHeadDim + k] = load1<F32>(y, (int64_t)j * step, h, k);
  }
}

// One wave per centroid: hi/lo planes of fp32(w*c) and the weighted norm.
__global__ __launch_bounds__(64) void k_prep(int C, const float* __restrict__ c,
                                             const float* __restrict__ w,
                                             uint16_t* __restrict__ planes, float* __restrict__ cn,
                                             int* __restrict__ amb_count) {
  const int h = blockIdx.x / C, j = blockIdx.x % C;
  const int lane = threadIdx.x;
  if (blockIdx.x == 0 && lane == 0 && amb_count) *amb_count = 0;
  const float* cr = c + ((int64_t)h * C + j) * kHeadDim;
  double nrm = 0.0;
  uint16_t* ph = planes + ((int64_t)h * 2 * C + j) * kHeadDim;
  uint16_t* pl = planes + ((int64_t)h * 2 * C + C + j) * kHeadDim;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int k = lane * 2 + e;
    const float cv = cr[k];
    const float wv = w ? w[h * kHeadDim + k] : 1.0f;
    const float b = wv * cv;
    const uint32_t hi = f32_to_bf16_bits(b);
    const uint32_t lo = f32_to_bf16_bits(b - bf16_bits_to_f32(hi));
    ph[k] = (uint16_t)hi;
    pl[k] = (uint16_t)lo;
    nrm += (double)wv * ((double)cv * (double)cv);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) nrm += __shfl_xor(nrm, off);
  if (lane == 0) cn[h * C + j] = (float)nrm;
}

template <bool F32>
__global__ __launch_bounds__(256) void k_assign(TensorView y, int C, int tiles_per_head, int n_heads,
                                                const uint16_t* __restrict__ planes,
                                                const float* __restrict__ cn,
                                                const float* __restrict__ w,
                                                uint8_t* __restrict__ labels, int* __restrict__ amb_count,
                                                int64_t* __restrict__ amb_list) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][2][32][kPitch];
  __shared__ float sCn[2][32];
  __shared__ __attribute__((aligned(16))) float sW[kHeadDim];
  const uint32_t logical = xcd_remap(blockIdx.x, (uint32_t)(tiles_per_head * n_heads));
  const int h = logical / tiles_per_head, tile = logical % tiles_per_head;
  const int N = (int)y.n_tokens;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  if (threadIdx.x < kHeadDim) sW[threadIdx.x] = w ? w[h * kHeadDim + threadIdx.x] : 1.0f;
  __syncthreads();

  // B operand (tokens): lane holds token `col` of sub-block t, channels s*16 + half*8 + [0, 8).
  // ynorm[t] accumulates sum_k w_k y_k^2 over the lane's channels (fp32; it only
  // sets the screening threshold).
  bf16x8 yh[2][8];
  bf16x8 yl[2][F32 ? 8 : 1];
  float ynorm[2] = {0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = tile * kAssignTokens + wave * 64 + t * 32 + col;
    const bool ok = tok < N;
    const int64_t base = (int64_t)(ok ? tok : 0) * y.stride_token + (int64_t)h * y.stride_head;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = s * 16 + half * 8;
      float v[8];
      if constexpr (F32) {
        const float* p = reinterpret_cast<const float*>(y.ptr) + base + ch;
        float4 a = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0, 0, 0, 0);
        float4 b = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0, 0, 0, 0);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        u16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hb = f32_to_bf16_bits(v[e]);
          hi[e] = (uint16_t)hb;
          lo[e] = (uint16_t)f32_to_bf16_bits(v[e] - bf16_bits_to_f32(hb));
        }
        yh[t][s] = __builtin_bit_cast(bf16x8, hi);
        yl[t][F32 ? s : 0] = __builtin_bit_cast(bf16x8, lo);
      } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(y.ptr) + base + ch;
        uint4 raw = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
        yh[t][s] = as_bf16x8(raw);
        const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((r4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
      const float4 w0 = *reinterpret_cast<const float4*>(&sW[ch]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sW[ch + 4]);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) ynorm[t] += wv[e] * (v[e] * v[e]);
    }
  }

  // top-2 of the screened values, branch-free; rows beyond C carry +inf.
  // Centroid planes stream through double-buffered LDS: the next block's
  // global loads are issued before the current block's MFMAs.
  float b1[2] = {INFINITY, INFINITY}, b2[2] = {INFINITY, INFINITY};
  int bidx[2] = {0, 0};
  const uint16_t* ph = planes + (int64_t)h * 2 * C * kHeadDim;
  const int nblk = (C + 31) / 32;
  uint4 pf[4];
  float cnpf = INFINITY;
  auto fetch = [&](int cb) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int v = threadIdx.x + x * 256;
      const int p = v >> 9, r = (v >> 4) & 31, c16 = v & 15;
      const int j = cb * 32 + r;
      pf[x] = make_uint4(0, 0, 0, 0);
      if (j < C) pf[x] = *reinterpret_cast<const uint4*>(ph + ((int64_t)p * C + j) * kHeadDim + c16 * 8);
    }
    if (threadIdx.x < 32) {
      const int j = cb * 32 + threadIdx.x;
      cnpf = j < C ? cn[h * C + j] : INFINITY;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int v = threadIdx.x + x * 256;
      const int p = v >> 9, r = (v >> 4) & 31, c16 = v & 15;
      *reinterpret_cast<uint4*>(&sA[buf][p][r][c16 * 8]) = pf[x];
    }
    if (threadIdx.x < 32) sCn[buf][threadIdx.x] = cnpf;
  };
  fetch(0);
  stash(0);
  __syncthreads();
  for (int cb = 0; cb < nblk; ++cb) {
    const int buf = cb & 1;
    if (cb + 1 < nblk) fetch(cb + 1);
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const uint4*>(&sA[buf][0][col][s * 16 + half * 8]));
      const bf16x8 alo = as_bf16x8(*reinterpret_cast<const uint4*>(&sA[buf][1][col][s * 16 + half * 8]));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yh[0][s], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yh[1][s], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, yh[0][s], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, yh[1][s], acc1, 0, 0, 0);
      if constexpr (F32) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yl[0][F32 ? s : 0], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, yl[1][F32 ? s : 0], acc1, 0, 0, 0);
      }
    }
    // Output layout: lane holds token `col`, centroid rows (r/4)*8 + half*4 + r%4
    // (increasing in r), so strict '<' keeps the lowest index among equal values.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jr = (r >> 2) * 8 + half * 4 + (r & 3);
      const int j = cb * 32 + jr;
      const float cnv = sCn[buf][jr];
      const float v0 = cnv - 2.0f * acc0[r];
      const float v1 = cnv - 2.0f * acc1[r];
      const bool l0 = v0 < b1[0], l1 = v1 < b1[1];
      b2[0] = l0 ? b1[0] : fminf(b2[0], v0);
      b2[1] = l1 ? b1[1] : fminf(b2[1], v1);
      bidx[0] = l0 ? j : bidx[0];
      bidx[1] = l1 ? j : bidx[1];
      b1[0] = l0 ? v0 : b1[0];
      b1[1] = l1 ? v1 : b1[1];
    }
    if (cb + 1 < nblk) stash(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float o1 = __shfl_xor(b1[t], 32), o2 = __shfl_xor(b2[t], 32);
    const int oi = __shfl_xor(bidx[t], 32);
    const float second = fminf(fmaxf(b1[t], o1), fminf(b2[t], o2));
    if (o1 < b1[t] || (o1 == b1[t] && oi < bidx[t])) { b1[t] = o1; bidx[t] = oi; }
    b2[t] = second;
    ynorm[t] += __shfl_xor(ynorm[t], 32);
  }

  // Close calls -- the two best screened values within the screening error
  // bound (generously 2e-5 of ||y||_w^2 + ||c||_w^2) -- are queued for k_refine,
  // which re-decides them from float64 distances.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = tile * kAssignTokens + wave * 64 + t * 32 + col;
    if (half == 0 && tok < N) {
      labels[(int64_t)h * N + tok] = (uint8_t)bidx[t];
      const float thr = 2e-5f * (ynorm[t] + cn[h * C + bidx[t]]);
      if (!(b2[t] - b1[t] > thr)) {
        const int slot = atomicAdd(amb_count, 1);
        amb_list[slot] = (int64_t)h * N + tok;
      }
    }
  }
}

// Float64 re-decision of queued close calls: one block per entry (grid-stride
// over the device-side count).  Thread j computes sum_k w_k (y_k - c_jk)^2 in
// channel order; the lowest index wins ties.
template <bool F32>
__global__ __launch_bounds__(256) void k_refine(TensorView y, int C, const float* __restrict__ cent,
                                                const float* __restrict__ w, const int* __restrict__ amb_count,
                                                const int64_t* __restrict__ amb_list, uint8_t* __restrict__ labels) {
  __shared__ float sY[kHeadDim];
  __shared__ float sW[kHeadDim];
  __shared__ double s_bv[4];
  __shared__ int s_bj[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = (int)y.n_tokens;
  const int count = *amb_count;
  for (int e = blockIdx.x; e < count; e += gridDim.x) {
    const int64_t ht = amb_list[e];
    const int h = (int)(ht / N), tok = (int)(ht % N);
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
      const int64_t off = (int64_t)tok * y.stride_token + (int64_t)h * y.stride_head + threadIdx.x;
      if constexpr (F32) sY[threadIdx.x] = reinterpret_cast<const float*>(y.ptr)[off];
      else sY[threadIdx.x] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(y.ptr)[off]);
      sW[threadIdx.x] = w ? w[h * kHeadDim + threadIdx.x] : 1.0f;
    }
    __syncthreads();
    const int j = threadIdx.x;
    double dist = INFINITY;
    if (j < C) {
      dist = 0.0;
      const float4* crow = reinterpret_cast<const float4*>(cent + ((int64_t)h * C + j) * kHeadDim);
      for (int kb = 0; kb < kHeadDim / 32; ++kb) {
        float4 cv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) cv[x] = crow[kb * 8 + x];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float c4[4] = {cv[x].x, cv[x].y, cv[x].z, cv[x].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = kb * 32 + x * 4 + q;
            const double diff = (double)sY[k] - (double)c4[q];
            dist = dist + (double)sW[k] * (diff * diff);
          }
        }
      }
    }
    double bv = dist;
    int bj = j;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oj = __shfl_xor(bj, off);
      if (ov < bv || (ov == bv && oj < bj)) { bv = ov; bj = oj; }
    }
    if (lane == 0) { s_bv[wave] = bv; s_bj[wave] = bj; }
    __syncthreads();
    if (threadIdx.x == 0) {
      double v = s_bv[0];
      int jj = s_bj[0];
      for (int x = 1; x < 4; ++x)
        if (s_bv[x] < v || (s_bv[x] == v && s_bj[x] < jj)) { v = s_bv[x]; jj = s_bj[x]; }
      labels[ht] = (uint8_t)jj;
    }
  }
}

// Counting sort of one head's tokens by label: counts, exclusive offsets and
// the member list (the order inside a cluster is immaterial: the sums below
// are exact up to ~2^-104).  One block of 1024 threads per head.
__global__ __launch_bounds__(1024) void k_sort(int N, int C, const uint8_t* __restrict__ labels,
                                               int32_t* __restrict__ start, int32_t* __restrict__ order,
                                               int32_t* __restrict__ counts, int* __restrict__ amb_count) {
  __shared__ int cnt[kMaxClusters];
  __shared__ int cur[kMaxClusters];
  const int h = blockIdx.x;
  if (h == 0 && threadIdx.x == 0 && amb_count) *amb_count = 0;   // the close-call queue of the next assign
  const uint8_t* lab = labels + (int64_t)h * N;
  for (int j = threadIdx.x; j < C; j += blockDim.x) cnt[j] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) atomicAdd(&cnt[min((int)lab[i], C - 1)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int j = 0; j < C; ++j) {
      cur[j] = acc;
      start[h * (C + 1) + j] = acc;
      acc += cnt[j];
    }
    start[h * (C + 1) + C] = acc;
  }
  __syncthreads();
  if (counts)
    for (int j = threadIdx.x; j < C; j += blockDim.x) counts[h * C + j] = cnt[j];
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int pos = atomicAdd(&cur[min((int)lab[i], C - 1)], 1);
    order[(int64_t)h * N + pos] = i;
  }
}

// One block per (head, cluster): the 4 waves take a quarter of the members
// each, accumulate rows in double-double (each lane two channels, up to 8 rows
// in flight), then combine in a fixed order.  The double-double value is the
// exact sum up to ~2^-104 relative, so its float64 rounding is the correctly
// rounded sum whatever the order; the mean is rounded once more to float32.
template <bool F32>
__global__ __launch_bounds__(256) void k_sum(TensorView y, int C, int n_heads, const int32_t* __restrict__ start,
                                             const int32_t* __restrict__ order, float* __restrict__ c,
                                             const float* __restrict__ w, uint16_t* __restrict__ planes,
                                             float* __restrict__ cn) {
  __shared__ double sd[4][64][4];
  const uint32_t logical = xcd_remap(blockIdx.x, (uint32_t)(n_heads * C));
  const int h = logical / C, j = logical % C;
  const int N = (int)y.n_tokens;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s0 = start[h * (C + 1) + j], s1 = start[h * (C + 1) + j + 1];
  const int n = s1 - s0;
  if (n == 0) return;                      // empty cluster: the centroid keeps its value
  const int per = (n + 3) / 4;
  const int m0 = s0 + wave * per, m1 = min(s1, m0 + per);
  const int32_t* ord = order + (int64_t)h * N;
  DD a0{0.0, 0.0}, a1{0.0, 0.0};
  const int64_t hoff = (int64_t)h * y.stride_head + lane * 2;
  int my_idx = 0;
  for (int m = m0; m < m1; m += 8) {
    if (((m - m0) & 63) == 0) my_idx = (m + lane < m1) ? ord[m + lane] : 0;   // 64 member ids per load
    float vx[8], vy[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      vx[q] = 0.f;
      vy[q] = 0.f;
      const int idq = __shfl(my_idx, ((m - m0) & 63) + q);
      if (m + q < m1) {
        const int64_t off = (int64_t)idq * y.stride_token + hoff;
        if constexpr (F32) {
          const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(y.ptr) + off);
          vx[q] = v.x;
          vy[q] = v.y;
        } else {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(y.ptr) + off);
          vx[q] = bf16_bits_to_f32(v & 0xFFFFu);
          vy[q] = bf16_bits_to_f32(v >> 16);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (m + q < m1) {
        a0.add((double)vx[q]);
        a1.add((double)vy[q]);
      }
    }
  }
  sd[wave][lane][0] = a0.hi;
  sd[wave][lane][1] = a0.lo;
  sd[wave][lane][2] = a1.hi;
  sd[wave][lane][3] = a1.lo;
  __syncthreads();
  if (wave == 0) {
    DD t0{sd[0][lane][0], sd[0][lane][1]}, t1{sd[0][lane][2], sd[0][lane][3]};
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      t0.add(DD{sd[w][lane][0], sd[w][lane][1]});
      t1.add(DD{sd[w][lane][2], sd[w][lane][3]});
    }
    float* cr = c + ((int64_t)h * C + j) * kHeadDim + lane * 2;
    const float c0 = (float)(t0.hi / (double)n);
    const float c1 = (float)(t1.hi / (double)n);
    cr[0] = c0;
    cr[1] = c1;
    if (planes) {   // operand planes and weighted norm for the next assign
      double nrm = 0.0;
      uint16_t* ph = planes + ((int64_t)h * 2 * C + j) * kHeadDim + lane * 2;
      uint16_t* pl = planes + ((int64_t)h * 2 * C + C + j) * kHeadDim + lane * 2;
      const float cv[2] = {c0, c1};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float wv = w ? w[h * kHeadDim + lane * 2 + e] : 1.0f;
        const float b = wv * cv[e];
        const uint32_t hi = f32_to_bf16_bits(b);
        ph[e] = (uint16_t)hi;
        pl[e] = (uint16_t)f32_to_bf16_bits(b - bf16_bits_to_f32(hi));
        nrm += (double)wv * ((double)cv[e] * (double)cv[e]);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) nrm += __shfl_xor(nrm, off);
      if (lane == 0) cn[h * C + j] = (float)nrm;
    }
  }
}

__global__ void k_centroid_bf16(int64_t n, const float* __restrict__ c, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint16_t)f32_to_bf16_bits(c[i]);
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_kmeans_init(const TensorView& y, int H, int C, float* c, hipStream_t s) {
  const dim3 grid((C + 7) / 8, H);
  if (y.dtype == 0) hipLaunchKernelGGL(k_init<true>, grid, dim3(256), 0, s, y, C, c);
  else hipLaunchKernelGGL(k_init<false>, grid, dim3(256), 0, s, y, C, c);
  return hipGetLastError();
}

hipError_t launch_centroid_prep(int H, int C, const float* c, const float* w, uint16_t* planes,
                                float* cn, int* amb_count, hipStream_t s) {
  hipLaunchKernelGGL(k_prep, dim3(H * C), dim3(64), 0, s, C, c, w, planes, cn, amb_count);
  return hipGetLastError();
}

hipError_t launch_kmeans_assign(const TensorView& y, int H, int C, const uint16_t* planes,
                                const float* cn, const float* c, const float* w, uint8_t* labels,
                                int* amb_count, int64_t* amb_list, hipStream_t s) {
  const int tiles = (int)((y.n_tokens + kAssignTokens - 1) / kAssignTokens);
  const dim3 grid(tiles * H);
  if (y.dtype == 0)
    hipLaunchKernelGGL(k_assign<true>, grid, dim3(256), 0, s, y, C, tiles, H, planes, cn, w, labels, amb_count,
                       amb_list);
  else
    hipLaunchKernelGGL(k_assign<false>, grid, dim3(256), 0, s, y, C, tiles, H, planes, cn, w, labels, amb_count,
                       amb_list);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rgrid(256);
  if (y.dtype == 0)
    hipLaunchKernelGGL(k_refine<true>, rgrid, dim3(256), 0, s, y, C, c, w, amb_count, amb_list, labels);
  else
    hipLaunchKernelGGL(k_refine<false>, rgrid, dim3(256), 0, s, y, C, c, w, amb_count, amb_list, labels);
  return hipGetLastError();
}

hipError_t launch_kmeans_update(const TensorView& y, int H, int C, const uint8_t* labels, float* c,
                                int32_t* counts, int32_t* start, int32_t* order, const float* w,
                                uint16_t* planes, float* cn, int* amb_count, hipStream_t s) {
  hipLaunchKernelGGL(k_sort, dim3(H), dim3(1024), 0, s, (int)y.n_tokens, C, labels, start, order, counts, amb_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(H * C);
  if (y.dtype == 0) hipLaunchKernelGGL(k_sum<true>, grid, dim3(256), 0, s, y, C, H, start, order, c, w, planes, cn);
  else hipLaunchKernelGGL(k_sum<false>, grid, dim3(256), 0, s, y, C, H, start, order, c, w, planes, cn);
  return hipGetLastError();
}

hipError_t launch_centroid_bf16(int H, int C, const float* c, uint16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)H * C * kHeadDim;
  hipLaunchKernelGGL(k_centroid_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, c, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u32(void* p, size_t n_words, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), (int64_t)n_words);
  return hipGetLastError();
}

}  // namespace qkv
