// Eigendecomposition of the history queries' second-moment matrices M_h
// (128 x 128, symmetric positive semi-definite), float64, on the GPU
// (QuantWM summary, "QuantWM", second technique: PSAC keeps the eigenvectors
// of the largest eigenvalues).
//
// Parallel cyclic Jacobi: one workgroup per head holds A = M_h in LDS.  A
// sweep is 127 steps of a round-robin schedule; each step pairs all 128
// indices into 64 disjoint pairs (p, q) and rotates every pair at once.  The
// rotation of a pair annihilates a_pq (tan 2 theta = 2 a_pq / (a_qq - a_pp),
// t = tan theta the smaller root, c = 1 / sqrt(1 + t^2), s = t c); as the
// pairs are disjoint their rotations commute, so A <- J^T A J is applied as
// one pass over the pairs' columns and then one over their rows, and the
// eigenvector matrix (kept transposed in global memory) as V^T <- J^T V^T,
// each column of V^T updated by one fixed thread throughout (no thread reads
// global memory that another thread of the block wrote).
// Sweeps stop when the off-diagonal mass is at most 1e-30 of the total (or
// after 60).  The eigenvalues are ranked in descending order (ties to the
// lower index); the leading `rank` eigenvectors and the energy fraction of
// their eigenvalues are written out.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

constexpr int kN = kHeadDim;         // 128
constexpr int kPairs = kN / 2;       // 64
constexpr int kEighThreads = 256;
constexpr int kEighMaxSweeps = 60;

// Step k of the round-robin over 128 indices: index 0 stays, 1 .. 127 rotate.
__device__ __forceinline__ void rr_pair(int k, int i, int& p, int& q) {
  int a, b;
  if (i == 0) {
    a = 0;
    b = 1 + k % (kN - 1);
  } else {
    a = 1 + (k + i) % (kN - 1);
    b = 1 + (k - i + (kN - 1)) % (kN - 1);
  }
  p = min(a, b);
  q = max(a, b);
}

// Block h: m [H][128][128] (row-major, read), vt [H][128][128] scratch,
// U [H][128][rank] (column b = eigenvector of the b-th largest eigenvalue),
// energy [H] (sum of the rank largest eigenvalues over their total; 0 when
// the total is not positive), diag [H][128] (M's own diagonal, as read).
__global__ __launch_bounds__(kEighThreads) void k_eigh(const double* __restrict__ m, double* __restrict__ vt,
                                                        int rank, float* __restrict__ U, float* __restrict__ energy,
                                                        double* __restrict__ diag) {
  __shared__ double A[kN][kN];
  __shared__ double rc[kPairs], rs[kPairs];
  __shared__ int rp[kPairs], rq[kPairs];
  __shared__ double red[kEighThreads / 64];
  __shared__ int rank_of[kN];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* mh = m + (int64_t)h * kN * kN;
  double* vh = vt + (int64_t)h * kN * kN;
  for (int i = tid; i < kN * kN; i += kEighThreads) A[i / kN][i % kN] = mh[i];
  if (tid < kN && diag) diag[(int64_t)h * kN + tid] = mh[tid * (kN + 1)];
  if (tid < kN)                                  // thread c owns column c of V^T
    for (int r = 0; r < kN; ++r) vh[r * kN + tid] = r == tid ? 1.0 : 0.0;
  __syncthreads();
  // sum over all elements (kind 0) or over the off-diagonal ones (kind 1), block-wide
  auto mass = [&](bool off_only) -> double {
    double v = 0.0;
    for (int i = tid; i < kN * kN; i += kEighThreads) {
      const int r = i / kN, c = i % kN;
      if (!off_only || r != c) v += A[r][c] * A[r][c];
    }
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kEighThreads / 64; ++w) t += red[w];
    return t;
  };
  const double total = mass(false);
  for (int sweep = 0; sweep < kEighMaxSweeps; ++sweep) {
    const double off = mass(true);               // block-uniform
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int k = 0; k < kN - 1; ++k) {
      if (tid < kPairs) {                        // the step's rotations
        int p, q;
        rr_pair(k, tid, p, q);
        const double apq = 0.5 * (A[p][q] + A[q][p]);
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (A[q][q] - A[p][p]) / (2.0 * apq);
          double t = 1.0 / (fabs(theta) + sqrt(theta * theta + 1.0));
          if (theta < 0.0) t = -t;
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        rp[tid] = p;
        rq[tid] = q;
        rc[tid] = c;
        rs[tid] = s;
      }
      __syncthreads();
      // columns p, q of every row: lanes take different pairs, the waves rows r = wave + 4 j
      {                                          // (the pairs are disjoint: eight rows' loads, then their stores)
        const int i = lane, p = rp[i], q = rq[i];
        const double c = rc[i], s = rs[i];
        for (int r0 = wave; r0 < kN; r0 += 8 * (kEighThreads / 64)) {
          double ap[8], aq[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            ap[u] = A[r0 + u * (kEighThreads / 64)][p];
            aq[u] = A[r0 + u * (kEighThreads / 64)][q];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            A[r0 + u * (kEighThreads / 64)][p] = c * ap[u] - s * aq[u];
            A[r0 + u * (kEighThreads / 64)][q] = s * ap[u] + c * aq[u];
          }
        }
      }
      __syncthreads();
      // rows p, q of every column: of V^T by threads 0 .. 127 (thread = column, every
      // pair, 32 pairs' loads at a time), of A by threads 128 .. 255 (16 at a time)
      if (tid < kN) {
        for (int i0 = 0; i0 < kPairs; i0 += 32) {
          double vp[32], vq[32];
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            vp[u] = vh[rp[i0 + u] * kN + tid];
            vq[u] = vh[rq[i0 + u] * kN + tid];
          }
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            const double c = rc[i0 + u], s = rs[i0 + u];
            vh[rp[i0 + u] * kN + tid] = c * vp[u] - s * vq[u];
            vh[rq[i0 + u] * kN + tid] = s * vp[u] + c * vq[u];
          }
        }
      } else {
        const int col = tid - kN;
        for (int i0 = 0; i0 < kPairs; i0 += 16) {
          double ap[16], aq[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            ap[u] = A[rp[i0 + u]][col];
            aq[u] = A[rq[i0 + u]][col];
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const double c = rc[i0 + u], s = rs[i0 + u];
            A[rp[i0 + u]][col] = c * ap[u] - s * aq[u];
            A[rq[i0 + u]][col] = s * ap[u] + c * aq[u];
          }
        }
      }
      __syncthreads();
    }
  }
  // descending order of the eigenvalues, ties to the lower index
  if (tid < kN) {
    const double d = A[tid][tid];
    int rk = 0;
    for (int j = 0; j < kN; ++j) {
      const double e = A[j][j];
      rk += (e > d || (e == d && j < tid)) ? 1 : 0;
    }
    rank_of[tid] = rk;
  }
  __syncthreads();
  // U[h][k][b] = V[k][j] for the j of rank b < rank (V^T row j is eigenvector j),
  // each thread reading its own column of V^T
  if (tid < kN) {
    for (int j = 0; j < kN; ++j) {
      const int b = rank_of[j];
      if (b < rank) U[((int64_t)h * kN + tid) * rank + b] = (float)vh[j * kN + tid];
    }
  }
  if (tid == 0 && energy) {
    double tot = 0.0, top = 0.0;
    for (int j = 0; j < kN; ++j) {
      tot += A[j][j];
      if (rank_of[j] < rank) top += A[j][j];
    }
    energy[h] = tot > 0.0 ? (float)(top / tot) : 0.0f;
  }
}

}  // namespace

hipError_t launch_eigh(const double* m, int H, double* vt, int rank, float* U, float* energy, double* diag,
                       hipStream_t s) {
  if (H < 1 || rank < 0 || rank > kN || (rank > 0 && !U)) return hipErrorInvalidValue;
  TimedLaunch tl_("k_eigh", s);
  hipLaunchKernelGGL(k_eigh, dim3((unsigned)H), dim3(kEighThreads), 0, s, m, vt, rank, U, energy, diag);
  return hipGetLastError();
}

}  // namespace qkv
