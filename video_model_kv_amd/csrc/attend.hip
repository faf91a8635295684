// Attention computed directly over the packed KV cache.
//
// Method: Quant VideoGen notes, "Key designs / Algorithm-system co-design"
// (quantization/dequantization fused with the attention kernel, 2-bit codes
// packed as integers) and "Method / Overall framework" (x_hat = S q + C_i);
// QuantWM summary, "QuantWM", second technique (PSAC: the stored projections of
// the key error on the query principal subspace U are added back to the logits,
// s += (q U) . coef).
//
// Work decomposition: one workgroup (4 waves, 256 threads) per (head, key
// split, 128-query tile).  A key split is a contiguous run of 64-key tiles of
// the concatenated chunks (a tile never straddles two chunks).  Per key tile the
// workgroup decodes K_hat and V_hat into LDS once for its 128 queries, then each
// wave (32 queries) computes S^T = K_hat Q^T and O^T += V_hat^T P^T on MFMA
// (v_mfma_f32_32x32x16_bf16) with an online softmax in the exp2 domain.
//
// Numerics: K_hat is formed in fp32 (exactly S q + C summed over stages in
// order) and split into bf16 hi + lo, both multiplied against the bf16 queries
// (fp32 queries are split too), so logits carry ~2^-17 relative operand error;
// V_hat and the probabilities enter P V in bf16 with fp32 accumulation.  The
// PSAC term rides one extra MFMA k-step: [coef | coef] against
// [hi(qU) | lo(qU)].  Splits are merged with the usual log-sum-exp rescaling.
#include "common.h"
#include "kernels.h"

namespace qkv {

namespace {

constexpr int kQTile = 128;     // queries per workgroup (4 waves x 32)
constexpr int kKTile = 64;      // keys per tile
constexpr int kKPitch = 136;    // bf16 pitch of the K_hat rows in LDS
constexpr int kVPitch = 68;     // bf16 pitch of the V_hat^T rows in LDS (34 dwords)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ const uint8_t* sp(const ChunkDecode& d, uint64_t off, uint64_t stride, int l) {
  return d.base + off + stride * (uint64_t)l;
}

__device__ __forceinline__ ChannelCode code_at(int p, int bits, int group, int n_int4, int int4_words) {
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

// Decode table of head h (block-cooperative; the caller synchronises).  A perm
// that is not a permutation decodes wrongly but stays inside every buffer.
__device__ __forceinline__ void build_tab(const ChunkDecode& d, int h, ChannelCode* tab) {
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) tab[p] = ChannelCode{0, 0, (uint8_t)d.bits, 0};
  __syncthreads();
  for (int p = threadIdx.x; p < kHeadDim; p += blockDim.x) {
    const int k = d.n_int4 > 0 ? ((int)(d.base + d.off_perm)[h * kHeadDim + p] & (kHeadDim - 1)) : p;
    tab[k] = code_at(p, d.bits, d.group, d.n_int4, d.int4_words);
  }
}

// Generic decode: x_hat of token j (within the chunk), channels k0..k0+NCH-1.
template <int NCH>
__device__ __forceinline__ void decode_generic(const ChunkDecode& d, const ChannelCode* tab, int h, int j,
                                               int k0, float* v) {
#pragma unroll
  for (int e = 0; e < NCH; ++e) v[e] = 0.0f;
  for (int l = 0; l < d.n_stages; ++l) {
    const int64_t row = (int64_t)h * d.N + j;
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(sp(d, d.off_codes, d.stage_codes, l)) + row * d.words;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(sp(d, d.off_scales, d.stage_scales, l)) + row * d.groups;
    const int lab = min((int)sp(d, d.off_labels, d.stage_labels, l)[row], d.C - 1);
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(sp(d, d.off_centroids, d.stage_centroids, l)) +
                           ((int64_t)h * d.C + lab) * kHeadDim + k0;
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const ChannelCode cc = tab[k0 + e];
      const uint32_t u = (codes[cc.word] >> cc.shift) & ((1u << cc.bits) - 1u);
      const float q = (float)((int)u - (1 << (cc.bits - 1)));
      const float yhat = __fadd_rn(bf16_bits_to_f32(scales[cc.group]) * q, bf16_bits_to_f32(crow[e]));
      v[e] = l == 0 ? yhat : __fadd_rn(v[e], yhat);
    }
  }
}

// Fast decode for one uniform INT2 stage with groups of >= 32 channels:
// channels k0..k0+NCH-1 (NCH <= 32, k0 % NCH == 0 and inside one group).
template <int NCH>
__device__ __forceinline__ void decode_int2(const ChunkDecode& d, int h, int j, int k0, float* v) {
  const int64_t row = (int64_t)h * d.N + j;
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(d.base + d.off_codes) + row * d.words + k0 / 16;
  const float S = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(d.base + d.off_scales)[row * d.groups + k0 / d.group]);
  const int lab = min((int)(d.base + d.off_labels)[row], d.C - 1);
  const uint16_t* crow = reinterpret_cast<const uint16_t*>(d.base + d.off_centroids) + ((int64_t)h * d.C + lab) * kHeadDim + k0;
  uint32_t w[(NCH + 15) / 16];
#pragma unroll
  for (int x = 0; x < (NCH + 15) / 16; ++x) w[x] = codes[x];
  uint4 cw[NCH / 8];
#pragma unroll
  for (int x = 0; x < NCH / 8; ++x) cw[x] = reinterpret_cast<const uint4*>(crow)[x];
  const uint32_t* cu = reinterpret_cast<const uint32_t*>(cw);
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    const uint32_t u = (w[e / 16] >> (2 * (e % 16))) & 3u;
    const float q = (float)((int)u - 2);
    const uint32_t cb = (cu[e / 2] >> (16 * (e & 1))) & 0xFFFFu;
    v[e] = __fadd_rn(S * q, bf16_bits_to_f32(cb));
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo_elem, float hi_elem) {
  return f32_to_bf16_bits(lo_elem) | (f32_to_bf16_bits(hi_elem) << 16);
}

template <bool QF32, bool KFAST, bool VFAST>
__global__ __launch_bounds__(256) void k_attend(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sKh[kKTile][kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sKl[kKTile][kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sKp[kKTile][16];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[kHeadDim][kVPitch];
  __shared__ ChannelCode tabK[kHeadDim], tabV[kHeadDim];

  const int q_tiles = (a.Nq + kQTile - 1) / kQTile;
  const uint32_t total = (uint32_t)(q_tiles * a.n_split * a.H);
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int qt = logical % q_tiles;
  const int split = (logical / q_tiles) % a.n_split;
  const int h = logical / (q_tiles * a.n_split);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kQTile + wave * 32 + col;     // this lane's query
  const bool qok = qrow < a.Nq;
  const int q_last = min(a.Nq, (qt + 1) * kQTile) - 1;

  // ---- Q fragments (B operand: column = query, k = channel) ----
  bf16x8 qh[8];
  bf16x8 ql[QF32 ? 8 : 1];
  {
    const int64_t base = (int64_t)(qok ? qrow : 0) * a.q.stride_token + (int64_t)h * a.q.stride_head;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = s * 16 + half * 8;
      if constexpr (QF32) {
        const float* p = reinterpret_cast<const float*>(a.q.ptr) + base + ch;
        float4 x0 = qok ? *reinterpret_cast<const float4*>(p) : make_float4(0, 0, 0, 0);
        float4 x1 = qok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0, 0, 0, 0);
        float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        u16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hb = f32_to_bf16_bits(v[e]);
          hi[e] = (uint16_t)hb;
          lo[e] = (uint16_t)f32_to_bf16_bits(v[e] - bf16_bits_to_f32(hb));
        }
        qh[s] = __builtin_bit_cast(bf16x8, hi);
        ql[QF32 ? s : 0] = __builtin_bit_cast(bf16x8, lo);
      } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(a.q.ptr) + base + ch;
        qh[s] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0));
      }
    }
  }
  bf16x8 qpsac;
  {
    u16x8 t;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.0f;
      if (a.psac_rank > 0 && qok && e < a.psac_rank) v = a.qu[((int64_t)h * a.Nq + qrow) * kMaxRank + e];
      const uint32_t hb = f32_to_bf16_bits(v);
      t[e] = (uint16_t)(half == 0 ? hb : f32_to_bf16_bits(v - bf16_bits_to_f32(hb)));
    }
    qpsac = __builtin_bit_cast(bf16x8, t);
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c2 = a.scale * kLog2e;

  const int t_begin = (int)(((int64_t)a.n_tiles * split) / a.n_split);
  const int t_end = (int)(((int64_t)a.n_tiles * (split + 1)) / a.n_split);
  // chunk holding tile t_begin (binary search over the tile starts)
  int c = 0;
  {
    int lo = 0, hi = a.n_chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.chunks[mid].tile_start <= t_begin) lo = mid; else hi = mid - 1;
    }
    c = lo;
  }
  int cur_chunk = -1;
  ChunkDecode dk, dv;
  for (int ti = t_begin; ti < t_end; ++ti) {
    while (c + 1 < a.n_chunks && a.chunks[c + 1].tile_start <= ti) ++c;
    const ChunkRec rec = a.chunks[c];
    const int token0 = (ti - rec.tile_start) * kKTile;
    const int64_t kstart = rec.token_start + token0;                     // global index of key 0
    // a tile wholly above the diagonal holds no visible key (visited anyway when
    // debug logits are requested, so that every masked entry is written)
    if (a.causal && kstart > q_last && !a.logits) continue;
    const int nvalid = min(kKTile, rec.n - token0);
    __syncthreads();   // previous tile fully consumed
    if (c != cur_chunk) {
      dk = make_decode(a.kp, rec.n, rec.kbase);
      dv = make_decode(a.vp, rec.n, rec.vbase);
      if constexpr (!KFAST) build_tab(dk, h, tabK);
      if constexpr (!VFAST) build_tab(dv, h, tabV);
      cur_chunk = c;
      __syncthreads();
    }
    // ---- decode K_hat (hi/lo) : thread = (key, 32-channel quarter) ----
    {
      const int key = threadIdx.x >> 2, k0 = (threadIdx.x & 3) * 32;
      float v[32];
      if (key < nvalid) {
        if constexpr (KFAST) decode_int2<32>(dk, h, token0 + key, k0, v);
        else decode_generic<32>(dk, tabK, h, token0 + key, k0, v);
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = 0.0f;
      }
      uint32_t hw[16], lw[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t h0 = f32_to_bf16_bits(v[2 * e]), h1 = f32_to_bf16_bits(v[2 * e + 1]);
        hw[e] = h0 | (h1 << 16);
        lw[e] = f32_to_bf16_bits(v[2 * e] - bf16_bits_to_f32(h0)) |
                (f32_to_bf16_bits(v[2 * e + 1] - bf16_bits_to_f32(h1)) << 16);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        *reinterpret_cast<uint4*>(&sKh[key][k0 + 8 * x]) = make_uint4(hw[4 * x], hw[4 * x + 1], hw[4 * x + 2], hw[4 * x + 3]);
        *reinterpret_cast<uint4*>(&sKl[key][k0 + 8 * x]) = make_uint4(lw[4 * x], lw[4 * x + 1], lw[4 * x + 2], lw[4 * x + 3]);
      }
      if (a.psac_rank > 0 && threadIdx.x < kKTile) {
        const int kk = threadIdx.x;
        uint16_t cf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cf[e] = 0;
        if (kk < nvalid) {
          const uint16_t* cp = reinterpret_cast<const uint16_t*>(dk.base + dk.off_psac) +
                               ((int64_t)h * dk.N + token0 + kk) * dk.psac_rank;
          for (int e = 0; e < dk.psac_rank; ++e) cf[e] = cp[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { sKp[kk][e] = cf[e]; sKp[kk][8 + e] = cf[e]; }
      }
    }
    // ---- decode V_hat^T (bf16) : thread = (key pair, 16-channel block) ----
    {
      const int kp = threadIdx.x & 31, k0 = (threadIdx.x >> 5) * 16;
      float v0[16], v1[16];
      const int j0 = 2 * kp, j1 = 2 * kp + 1;
      if (j0 < nvalid) {
        if constexpr (VFAST) decode_int2<16>(dv, h, token0 + j0, k0, v0);
        else decode_generic<16>(dv, tabV, h, token0 + j0, k0, v0);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v0[e] = 0.0f;
      }
      if (j1 < nvalid) {
        if constexpr (VFAST) decode_int2<16>(dv, h, token0 + j1, k0, v1);
        else decode_generic<16>(dv, tabV, h, token0 + j1, k0, v1);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v1[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        *reinterpret_cast<uint32_t*>(&sVt[k0 + e][2 * kp]) = pack_bf16x2(v0[e], v1[e]);
    }
    __syncthreads();

    // ---- S^T = K_hat Q^T for the two 32-key blocks ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = {};
      const int krow = kb * 32 + col;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kh = as_bf16x8(*reinterpret_cast<const uint4*>(&sKh[krow][s * 16 + half * 8]));
        const bf16x8 kl = as_bf16x8(*reinterpret_cast<const uint4*>(&sKl[krow][s * 16 + half * 8]));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[s], acc, 0, 0, 0);
        if constexpr (QF32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[QF32 ? s : 0], acc, 0, 0, 0);
      }
      if (a.psac_rank > 0) {
        const bf16x8 kp = as_bf16x8(*reinterpret_cast<const uint4*>(&sKp[krow][half * 8]));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kp, qpsac, acc, 0, 0, 0);
      }
      sacc[kb] = acc;
    }

    // ---- masks, debug logits, online softmax (exp2 domain) ----
    float x[2][16];
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);   // key within tile
        const int64_t kg = kstart + kl;
        bool valid = kl < nvalid;
        if (a.causal) valid = valid && (kg <= qrow);
        if (a.logits && qok && kl < nvalid)
          a.logits[((int64_t)h * a.Nq + qrow) * a.Nk + kg] = valid ? sacc[kb][r] * a.scale : -INFINITY;
        const float xv = valid ? sacc[kb][r] * c2 : -INFINITY;
        x[kb][r] = xv;
        mloc = fmaxf(mloc, xv);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    float alpha = 1.0f;
    if (m_new != -INFINITY) alpha = exp2f(m_run - m_new);   // m_run = -inf gives 0
    float psum = 0.0f;
    u16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = (m_new == -INFINITY) ? 0.0f : exp2f(x[kb][r] - m_new);
        psum += p;
        pb[kb][r >> 3][r & 7] = (uint16_t)f32_to_bf16_bits(p);
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;

    // ---- O^T += V_hat^T P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pfrag = __builtin_bit_cast(bf16x8, pb[kb][t]);
        const int kbase = kb * 32 + t * 16 + half * 4;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int drow = db * 32 + col;
          const uint2 v0 = *reinterpret_cast<const uint2*>(&sVt[drow][kbase]);
          const uint2 v1 = *reinterpret_cast<const uint2*>(&sVt[drow][kbase + 8]);
          const bf16x8 vfrag = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag, pfrag, o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qok) return;
  if (a.n_split == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* orow = a.out + (int64_t)qrow * a.out_stride_token + (int64_t)h * a.out_stride_head;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        *reinterpret_cast<float4*>(orow + d0) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      }
  } else {
    float* prow = a.part_o + (((int64_t)split * a.H + h) * a.Nq + qrow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        *reinterpret_cast<float4*>(prow + d0) = make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
      }
    if (half == 0) {
      float* ml = a.part_ml + (((int64_t)split * a.H + h) * a.Nq + qrow) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Merge the splits: thread = (head, query, 4 channels).
__global__ __launch_bounds__(256) void k_merge(AttendArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.H * a.Nq * (kHeadDim / 4);
  if (gid >= total) return;
  const int d0 = (int)(gid % (kHeadDim / 4)) * 4;
  const int64_t hq = gid / (kHeadDim / 4);
  const int qrow = (int)(hq % a.Nq), h = (int)(hq / a.Nq);
  float mmax = -INFINITY;
  for (int s = 0; s < a.n_split; ++s)
    mmax = fmaxf(mmax, a.part_ml[(((int64_t)s * a.H + h) * a.Nq + qrow) * 2]);
  float4 acc = make_float4(0, 0, 0, 0);
  float lsum = 0.0f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const int64_t r = ((int64_t)s * a.H + h) * a.Nq + qrow;
      const float ms = a.part_ml[r * 2];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - mmax);
      lsum += wgt * a.part_ml[r * 2 + 1];
      const float4 v = *reinterpret_cast<const float4*>(a.part_o + r * kHeadDim + d0);
      acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float* orow = a.out + (int64_t)qrow * a.out_stride_token + (int64_t)h * a.out_stride_head + d0;
  *reinterpret_cast<float4*>(orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// qU[h][i][b] = sum_k q_ik U[h][k][b] (float64 accumulation, rounded to fp32).
template <bool QF32>
__global__ __launch_bounds__(256) void k_qu(TensorView q, int H, int Nq, int r, const float* __restrict__ U,
                                            float* __restrict__ qu) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)H * Nq) return;
  const int i = (int)(gid % Nq), h = (int)(gid / Nq);
  double acc[kMaxRank];
#pragma unroll
  for (int b = 0; b < kMaxRank; ++b) acc[b] = 0.0;
  const int64_t base = (int64_t)i * q.stride_token + (int64_t)h * q.stride_head;
  for (int k = 0; k < kHeadDim; ++k) {
    float qv;
    if constexpr (QF32) qv = reinterpret_cast<const float*>(q.ptr)[base + k];
    else qv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q.ptr)[base + k]);
#pragma unroll
    for (int b = 0; b < kMaxRank; ++b)
      if (b < r) acc[b] += (double)qv * (double)U[((int64_t)h * kHeadDim + k) * r + b];
  }
#pragma unroll
  for (int b = 0; b < kMaxRank; ++b) qu[gid * kMaxRank + b] = b < r ? (float)acc[b] : 0.0f;
}

__global__ void k_upload(ChunkBatch b, ChunkRec* __restrict__ dst) {
  const int i = threadIdx.x;
  if (i < b.count) dst[b.first + i] = b.rec[i];
}

}  // namespace

hipError_t launch_upload_chunks(const ChunkBatch& b, ChunkRec* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_upload, dim3(1), dim3(kChunkBatch), 0, s, b, dst);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.psac_rank > 0) {
    const int64_t n = (int64_t)a.H * a.Nq;
    if (a.q.dtype == 0)
      hipLaunchKernelGGL(k_qu<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.q, a.H, a.Nq, a.psac_rank, a.U, a.qu);
    else
      hipLaunchKernelGGL(k_qu<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.q, a.H, a.Nq, a.psac_rank, a.U, a.qu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int q_tiles = (a.Nq + kQTile - 1) / kQTile;
  const dim3 grid((unsigned)(q_tiles * a.n_split * a.H));
  const bool kf = a.k_uniform_int2_1stage;
  const bool vf = a.v_uniform_int2_1stage;
#define QKV_AT(QF, KF, VF) hipLaunchKernelGGL((k_attend<QF, KF, VF>), grid, dim3(256), 0, s, a)
  if (a.q.dtype == 0) {
    if (kf && vf) QKV_AT(true, true, true);
    else if (!kf && vf) QKV_AT(true, false, true);
    else if (kf && !vf) QKV_AT(true, true, false);
    else QKV_AT(true, false, false);
  } else {
    if (kf && vf) QKV_AT(false, true, true);
    else if (!kf && vf) QKV_AT(false, false, true);
    else if (kf && !vf) QKV_AT(false, true, false);
    else QKV_AT(false, false, false);
  }
#undef QKV_AT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t total = (int64_t)a.H * a.Nq * (kHeadDim / 4);
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qkv
