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
// pairs are disjoint their rotations commute, so A <- J^T A J is applied in
// one pass over the 2 x 2 blocks that the pairs cut A into.
// Sweeps stop when the off-diagonal mass is at most 1e-30 of the total (or
// after the sweeps the rotation record has room for, at most 60).  The
// eigenvalues are ranked in descending order (ties to the lower index).
// Eigenvectors: the eigenvector matrix is V = J_1 J_2 ... J_n, and only its
// columns of the `rank` (at most 8) largest eigenvalues are wanted, so the
// sweeps record every step's (c, s) and the columns are formed at the end as
// J_1 (J_2 (... (J_n e_j))), the recorded steps applied backwards to unit
// vectors in LDS.  Those columns, and the energy fraction of their
// eigenvalues, are written out.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace qkv {

namespace {

constexpr int kN = kHeadDim;         // 128
constexpr int kPairs = kN / 2;       // 64
constexpr int kSteps = kN - 1;       // 127 steps per sweep
constexpr int kEighThreads = 1024;
constexpr int kEighWaves = kEighThreads / 64;
constexpr int kRowPairsPerWave = kPairs / kEighWaves;   // 4
constexpr int kEighMaxSweeps = 60;
constexpr size_t kSweepRecordBytes = (size_t)kSteps * kPairs * 16;   // (c, s) per pair and step

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

// Block h: m [H][128][128] (row-major, read), rot [H][max_sweeps][127][64] (c, s)
// scratch, U [H][128][rank] (column b = eigenvector of the b-th largest
// eigenvalue), energy [H] (sum of the rank largest eigenvalues over their total;
// 0 when the total is not positive), diag [H][128] (M's own diagonal, as read).
__global__ __launch_bounds__(kEighThreads) void k_eigh(const double* __restrict__ m, double2* __restrict__ rot,
                                                        int max_sweeps, int rank, float* __restrict__ U,
                                                        float* __restrict__ energy, double* __restrict__ diag) {
  __shared__ double A[kN][kN];
  __shared__ double rc[kPairs], rs[kPairs];
  __shared__ int rp[kPairs], rq[kPairs];
  __shared__ double red[kEighThreads / 64];
  __shared__ int rank_of[kN];
  __shared__ int sel[kMaxRank];
  __shared__ double X[kMaxRank][kN];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* mh = m + (int64_t)h * kN * kN;
  double2* rh = rot + (int64_t)h * max_sweeps * kSteps * kPairs;
  for (int i = tid; i < kN * kN; i += kEighThreads) A[i / kN][i % kN] = mh[i];
  if (tid < kN && diag) diag[(int64_t)h * kN + tid] = mh[tid * (kN + 1)];
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
  int n_sweeps = 0;                              // block-uniform
  for (; n_sweeps < max_sweeps; ++n_sweeps) {
    const double off = mass(true);               // block-uniform
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int k = 0; k < kSteps; ++k) {
      if (tid < kPairs) {                        // the step's rotations, recorded by the thread that forms them
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
        rh[((int64_t)n_sweeps * kSteps + k) * kPairs + tid] = make_double2(c, s);
      }
      __syncthreads();
      // J^T A J over the 64 x 64 blocks of the pairs: block (i, j) holds rows p_i, q_i and
      // columns p_j, q_j, which no other block touches, so each block is read once, its
      // columns rotated by pair j and then its rows by pair i (the operations of a pass
      // over the columns followed by one over the rows), and written once.  Lane = column
      // pair j, each wave 4 row pairs, all their blocks' loads ahead of their stores.
      {
        const int pj = rp[lane], qj = rq[lane];
        const double cj = rc[lane], sj = rs[lane];
        {
          const int i0 = wave * kRowPairsPerWave;
          double a[kRowPairsPerWave][4];
#pragma unroll
          for (int u = 0; u < kRowPairsPerWave; ++u) {
            const int pi = rp[i0 + u], qi = rq[i0 + u];
            a[u][0] = A[pi][pj];
            a[u][1] = A[pi][qj];
            a[u][2] = A[qi][pj];
            a[u][3] = A[qi][qj];
          }
#pragma unroll
          for (int u = 0; u < kRowPairsPerWave; ++u) {
            const int pi = rp[i0 + u], qi = rq[i0 + u];
            const double ci = rc[i0 + u], si = rs[i0 + u];
            const double x0 = cj * a[u][0] - sj * a[u][1], x1 = sj * a[u][0] + cj * a[u][1];   // row p_i
            const double y0 = cj * a[u][2] - sj * a[u][3], y1 = sj * a[u][2] + cj * a[u][3];   // row q_i
            A[pi][pj] = ci * x0 - si * y0;
            A[qi][pj] = si * x0 + ci * y0;
            A[pi][qj] = ci * x1 - si * y1;
            A[qi][qj] = si * x1 + ci * y1;
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
    if (rk < rank) sel[rk] = tid;                // the ranks are a permutation of 0 .. 127
  }
  __syncthreads();
  if (tid == 0 && energy) {
    double tot = 0.0, top = 0.0;
    for (int j = 0; j < kN; ++j) {
      tot += A[j][j];
      if (rank_of[j] < rank) top += A[j][j];
    }
    energy[h] = tot > 0.0 ? (float)(top / tot) : 0.0f;
  }
  // U[h][k][b] = V[k][sel[b]]: wave 0 applies the recorded steps, last first, to the
  // unit vectors e_sel[b]; lane i takes pair slot i of every step, whose (c, s) this
  // same thread recorded, and the wave orders its LDS accesses between steps
  if (wave == 0 && rank > 0) {
#pragma unroll
    for (int b = 0; b < kMaxRank; ++b)
      if (b < rank) {
        X[b][lane] = lane == sel[b] ? 1.0 : 0.0;
        X[b][lane + kPairs] = lane + kPairs == sel[b] ? 1.0 : 0.0;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the records are read kAhead steps at a time, the next batch in flight while
    // the current one is applied
    constexpr int kAhead = 8;
    auto load_batch = [&](int st0, double2* dst) {
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        dst[u] = st0 - u >= 0 ? rh[(int64_t)(st0 - u) * kPairs + lane] : make_double2(1.0, 0.0);
    };
    double2 cur[kAhead];
    load_batch(n_sweeps * kSteps - 1, cur);
    for (int st0 = n_sweeps * kSteps - 1; st0 >= 0; st0 -= kAhead) {
      double2 nxt[kAhead];
      load_batch(st0 - kAhead, nxt);
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int st = st0 - u;                  // wave-uniform
        if (st < 0) break;
        int p, q;
        rr_pair(st % kSteps, lane, p, q);
#pragma unroll
        for (int b = 0; b < kMaxRank; ++b)
          if (b < rank) {
            const double xp = X[b][p], xq = X[b][q];
            X[b][p] = cur[u].x * xp + cur[u].y * xq;     // x <- J x: J_pp = J_qq = c, J_pq = s, J_qp = -s
            X[b][q] = cur[u].x * xq - cur[u].y * xp;
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll
      for (int u = 0; u < kAhead; ++u) cur[u] = nxt[u];
    }
#pragma unroll
    for (int b = 0; b < kMaxRank; ++b)
      if (b < rank) {
        U[((int64_t)h * kN + lane) * rank + b] = (float)X[b][lane];
        U[((int64_t)h * kN + lane + kPairs) * rank + b] = (float)X[b][lane + kPairs];
      }
  }
}

}  // namespace

hipError_t launch_eigh(const double* m, int H, void* rot, size_t rot_bytes, int rank, float* U, float* energy,
                       double* diag, hipStream_t s) {
  if (H < 1 || rank < 0 || rank > kMaxRank || (rank > 0 && !U) || !rot) return hipErrorInvalidValue;
  const size_t room = rot_bytes / ((size_t)H * kSweepRecordBytes);
  if (room < 1) return hipErrorInvalidValue;
  const int max_sweeps = (int)std::min<size_t>(room, kEighMaxSweeps);
  TimedLaunch tl_("k_eigh", s);
  hipLaunchKernelGGL(k_eigh, dim3((unsigned)H), dim3(kEighThreads), 0, s, m, reinterpret_cast<double2*>(rot),
                     max_sweeps, rank, U, energy, diag);
  return hipGetLastError();
}

}  // namespace qkv
