// libqkv host side: argument validation, packed-chunk layout, workspace
// planning and launch sequencing of the C-ABI declared in include/qkv.h.
//
// Everything here runs before any work is enqueued, so each error path is
// reachable without a GPU.  The library holds no device state: all device
// memory is caller-owned (packed chunks, workspace, outputs).
#include "qkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "kernels.h"

using namespace qkv;

namespace qkv {

bool mix4_order(const LayoutParams& p, MixOrder* m) {
  const int n4 = p.n_int4, g = p.group;
  if (n4 <= 0 || (n4 & 1) || (g & 1) || p.bits != 2) return false;
  // groups in storage order: the 4-bit class, then the 2-bit class, runs of g
  int start[kHeadDim], len[kHeadDim], ng = 0;
  for (int a = 0; a < n4; a += g) { start[ng] = a; len[ng] = std::min(g, n4 - a); ++ng; }
  for (int a = 0; a < kHeadDim - n4; a += g) { start[ng] = n4 + a; len[ng] = std::min(g, kHeadDim - n4 - a); ++ng; }
  if (ng > kMix4MaxGroups) return false;
  int pos = 0, grp[kHeadDim];
  for (int k = 0; k < ng; ++k)                   // whole 8-position items of each group
    for (int b = 0; b + 8 <= len[k]; b += 8)
      for (int t = 0; t < 8; ++t) { m->rho[pos] = (uint8_t)(start[k] + b + t); grp[pos++] = k; }
  for (int k = 0; k < ng; ++k)                   // then the groups' remainders, in group order
    for (int t = len[k] / 8 * 8; t < len[k]; ++t) { m->rho[pos] = (uint8_t)(start[k] + t); grp[pos++] = k; }
  if (pos != kHeadDim) return false;
  for (int it = 0; it < 16; ++it) {
    const int* gi = grp + it * 8;
    int jb = 4;
    for (int t = 1; t < 8; ++t) {
      if (gi[t] == gi[t - 1]) continue;
      if (jb != 4 || (t & 1)) return false;      // a second split, or a split inside a pair
      jb = t / 2;
    }
    m->glo[it] = (uint8_t)gi[0];
    m->ghi[it] = (uint8_t)gi[7];
    m->jb[it] = (uint8_t)jb;
  }
  return true;
}

}  // namespace qkv

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return QKV_OK;
}

#define QKV_HIP(expr)                                                                 \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess) return fail(QKV_EDEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define QKV_TRY(expr)           \
  do {                          \
    int st_ = (expr);           \
    if (st_ != QKV_OK) return st_; \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_config(const qkv_config* c, const char* what) {
  if (!c) return fail(QKV_EINVAL, "%s: config is NULL", what);
  if (c->head_dim != kHeadDim)
    return fail(QKV_EUNSUPPORTED, "%s: head_dim %d (the library supports 128)", what, c->head_dim);
  if (c->n_heads < 1 || c->n_heads > 1024) return fail(QKV_EINVAL, "%s: n_heads %d not in [1, 1024]", what, c->n_heads);
  if (c->n_clusters < 1 || c->n_clusters > kMaxClusters)
    return fail(QKV_EINVAL, "%s: n_clusters %d not in [1, 256]", what, c->n_clusters);
  if (c->kmeans_iters < 1 || c->kmeans_iters > 1000)
    return fail(QKV_EINVAL, "%s: kmeans_iters %d not in [1, 1000]", what, c->kmeans_iters);
  if (c->n_stages < 1 || c->n_stages > kMaxStages)
    return fail(QKV_EINVAL, "%s: n_stages %d not in [1, %d]", what, c->n_stages, kMaxStages);
  if (c->bits != 2 && c->bits != 4) return fail(QKV_EINVAL, "%s: bits %d (2 or 4)", what, c->bits);
  if (c->group != 16 && c->group != 32 && c->group != 64 && c->group != 128)
    return fail(QKV_EINVAL, "%s: group %d must be a multiple of 16 dividing 128", what, c->group);
  if (c->n_int4_channels < 0 || c->n_int4_channels >= kHeadDim)
    return fail(QKV_EINVAL, "%s: n_int4_channels %d not in [0, 127]", what, c->n_int4_channels);
  if (c->n_int4_channels > 0 && c->bits != 2)
    return fail(QKV_EINVAL, "%s: the mixed layout needs bits == 2 for the base class", what);
  if (c->psac_rank < 0 || c->psac_rank > kMaxRank)
    return fail(QKV_EINVAL, "%s: psac_rank %d not in [0, 8]", what, c->psac_rank);
  if (c->use_qsac < 0 || c->use_qsac > 2) return fail(QKV_EINVAL, "%s: use_qsac must be 0, 1 or 2", what);
  if (c->flags & ~QKV_FLAG_RTN) return fail(QKV_EINVAL, "%s: unknown flags 0x%x", what, c->flags);
  return QKV_OK;
}

LayoutParams params_of(const qkv_config* c) {
  LayoutParams p;
  p.H = c->n_heads;
  p.C = c->n_clusters;
  p.n_stages = c->n_stages;
  p.bits = c->bits;
  p.group = c->group;
  p.n_int4 = c->n_int4_channels;
  p.psac_rank = c->psac_rank;
  return p;
}

ChunkDecode decode_of(const qkv_config* c, int64_t n, const void* base) {
  return make_decode(params_of(c), n, base);
}

void layout_of(const qkv_config* c, int64_t n, qkv_layout* L) {
  const ChunkDecode d = decode_of(c, n, nullptr);
  std::memset(L, 0, sizeof *L);
  L->bytes = d.bytes;
  L->off_codes = d.off_codes;
  L->stage_bytes_codes = d.stage_codes;
  L->off_scales = d.off_scales;
  L->stage_bytes_scales = d.stage_scales;
  L->off_labels = d.off_labels;
  L->stage_bytes_labels = d.stage_labels;
  L->off_centroids = d.off_centroids;
  L->stage_bytes_centroids = d.stage_centroids;
  L->off_perm = d.off_perm;
  L->off_psac = d.off_psac;
  L->words_per_token = d.words;
  L->groups_per_token = d.groups;
  L->int4_words = d.int4_words;
  L->n_tokens = n;
}

int check_tensor(const qkv_tensor* t, int n_heads, const char* what, bool allow_f32 = true) {
  if (!t) return fail(QKV_EINVAL, "%s: tensor is NULL", what);
  if (!t->ptr) return fail(QKV_EINVAL, "%s: data pointer is NULL", what);
  if (!aligned16(t->ptr)) return fail(QKV_EINVAL, "%s: data pointer not 16-byte aligned", what);
  if (t->dtype != QKV_F32 && t->dtype != QKV_BF16) return fail(QKV_EINVAL, "%s: dtype %d", what, t->dtype);
  if (!allow_f32 && t->dtype == QKV_F32) return fail(QKV_EUNSUPPORTED, "%s: f32 not supported here", what);
  if (t->n_tokens < 1 || t->n_tokens > (int64_t)1 << 24) return fail(QKV_EINVAL, "%s: n_tokens %lld", what, (long long)t->n_tokens);
  if (t->stride_token < 0 || t->stride_head < 0 || t->stride_token % 8 || t->stride_head % 8)
    return fail(QKV_EINVAL, "%s: strides must be non-negative multiples of 8 elements", what);
  if (n_heads > 1 && t->stride_head < kHeadDim)
    return fail(QKV_EINVAL, "%s: head stride %lld overlaps the channel dimension", what, (long long)t->stride_head);
  if (t->n_tokens > 1 && t->stride_token < kHeadDim)
    return fail(QKV_EINVAL, "%s: token stride %lld overlaps the channel dimension", what, (long long)t->stride_token);
  return QKV_OK;
}

TensorView view_of(const qkv_tensor* t) {
  TensorView v;
  v.ptr = t->ptr;
  v.dtype = t->dtype == QKV_F32 ? 0 : 1;
  v.n_tokens = t->n_tokens;
  v.stride_token = t->stride_token;
  v.stride_head = t->stride_head;
  return v;
}

// ---- workspace plans ----
struct QuantWs {
  uint64_t c, amb_count, grp_off, grp_list, ynorm, wq, rpart, dsum, dcnt, emag, cert, hlist, prev, ybuf0, ybuf1, bytes;
};

QuantWs quant_ws(const qkv_config* c, int64_t n) {
  const uint64_t H = c->n_heads, C = c->n_clusters;
  QuantWs w;
  uint64_t off = 0;
  w.c = off;       off += align256(H * C * kHeadDim * 4);
  w.amb_count = off; off += 256;
  w.grp_off = off; off += align256(H * (C + 1) * 4);
  w.grp_list = off; off += align256(H * (uint64_t)n * 2);
  w.ynorm = off;   off += align256(H * (uint64_t)n * 4);                 // ||y||^2 kept across iterations
  w.wq = off;      off += align256(H * kHeadDim * 4);                  // QSAC weights with the range factor
  w.rpart = off;   off += align256(H * kRangeSplits * 2 * kHeadDim * 4);
  // incremental k-means updates (grouped heads): exact sums, counts, magnitude
  // range, labels of the last two updates
  const bool inc = n <= kGroupMaxTokens;
  w.dsum = off;    if (inc) off += align256(H * C * kHeadDim * 8);
  w.dcnt = off;    if (inc) off += align256(H * C * 4);
  w.emag = off;    if (inc) off += align256(H * 2 * kHeadDim * 4);
  w.cert = off;    if (inc) off += align256(H * 4);
  w.hlist = off;   if (inc) off += align256((2 + 2 * H) * 4);
  w.prev = off;    if (inc) off += align256(2 * H * (uint64_t)n);
  w.ybuf0 = off;   if (c->n_stages > 1) off += align256(H * (uint64_t)n * kHeadDim * 4);
  w.ybuf1 = off;   if (c->n_stages > 2) off += align256(H * (uint64_t)n * kHeadDim * 4);
  w.bytes = off;
  return w;
}

constexpr int kTileKeys = 64;

struct AttendWs {
  uint64_t chunks, tiles, qu, part_o, part_ml, k16, v16, range, mix, krep, dense, bytes;
};

// rows = n_split * nq: one partial (o, m, l) row per split and query (none when n_split == 1);
// kC16 / vC16: clusters of the key / value tables copied to fp16 for the fast decode (0: none)
// krep_bytes: mix4 codes of the keys (64 bytes per token-head), 0 when the keys take another path
// dense_bytes: the dense fp16 K and V rows of a cache on the generic decode (0: none)
AttendWs attend_ws(int H, int64_t nq, int n_chunks, int64_t n_tiles, int64_t split_rows, int kC16, int vC16,
                   uint64_t krep_bytes, uint64_t dense_bytes = 0) {
  AttendWs w;
  uint64_t off = 0;
  w.chunks = off;  off += align256((uint64_t)n_chunks * sizeof(ChunkRec));
  w.tiles = off;   off += align256((uint64_t)n_tiles * sizeof(TileRec));
  w.qu = off;      off += align256((uint64_t)H * nq * kMaxRank * 4);
  w.part_o = off;  off += align256((uint64_t)split_rows * H * kHeadDim * 4);
  w.part_ml = off; off += align256((uint64_t)split_rows * H * 2 * 4);
  w.k16 = off;     off += align256((uint64_t)n_chunks * H * kC16 * kHeadDim * 2);
  w.v16 = off;     off += align256((uint64_t)n_chunks * H * vC16 * kHeadDim * 2);
  w.range = off;   off += 256;
  w.mix = off;     off += align256(sizeof(MixOrder));
  w.krep = off;    off += align256(krep_bytes);
  w.dense = off;   off += align256(dense_bytes);
  w.bytes = off;
  return w;
}

// Key splits.  One attention workgroup fills a compute unit (its LDS use), so
// the grid runs in rounds of kComputeUnits workgroups.  The split count is at
// most split_cap (about eight rounds of workgroups; the workspace is sized for
// it) and minimises rounds x (tiles per split + ~3 tiles of fixed per-split
// cost: pipeline fill and the partial write).
constexpr int kComputeUnits = 256;

int split_cap(int H, int64_t nq) {
  const int64_t base = (nq + kAttendQueries - 1) / kAttendQueries * H;
  return (int)std::max<int64_t>(1, std::min<int64_t>(64, (8 * kComputeUnits + base - 1) / base));
}

int choose_splits(int H, int64_t nq, int64_t n_tiles) {
  const int64_t base = (nq + kAttendQueries - 1) / kAttendQueries * H;
  const int64_t hi = std::max<int64_t>(1, std::min<int64_t>(n_tiles, split_cap(H, nq)));
  int64_t best = 1;
  double best_cost = 0.0;
  for (int64_t s = 1; s <= hi; ++s) {
    const int64_t rounds = (base * s + kComputeUnits - 1) / kComputeUnits;
    const double cost = (double)rounds * ((double)n_tiles / (double)s + 3.0);
    if (s == 1 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return (int)best;
}

// The largest n_split * nq over every query count nq <= n_query (split counts
// never exceed split_cap(H, nq), which only changes with the number of query tiles).
int64_t max_tiles(int64_t max_chunk_tokens, int n_chunks) {
  return (int64_t)n_chunks * ((max_chunk_tokens + kTileKeys - 1) / kTileKeys);
}

int64_t max_split_rows(int H, int64_t n_query) {
  int64_t best = 0;
  const int64_t tiles = (n_query + kAttendQueries - 1) / kAttendQueries;
  for (int64_t k = 1; k <= tiles; ++k) {
    const int64_t nq = std::min<int64_t>(n_query, k * kAttendQueries);
    const int cap = split_cap(H, nq);
    best = std::max<int64_t>(best, cap > 1 ? cap * nq : 0);
    if (cap == 1) break;                     // from here on no splits at all
  }
  return best;
}

constexpr int kGramSplit = 16;

uint64_t psac_ws(int H) {
  return align256((uint64_t)kGramSplit * H * kHeadDim * kHeadDim * 8) + align256((uint64_t)H * kHeadDim * kHeadDim * 8);
}

int check_ws(const void* ws, size_t have, uint64_t need, const char* what) {
  if (need == 0) return QKV_OK;
  if (!ws) return fail(QKV_EWORKSPACE, "%s: workspace is NULL (%llu bytes needed)", what, (unsigned long long)need);
  if (!aligned16(ws)) return fail(QKV_EINVAL, "%s: workspace not 16-byte aligned", what);
  if (have < need)
    return fail(QKV_EWORKSPACE, "%s: workspace has %zu bytes, %llu needed", what, have, (unsigned long long)need);
  return QKV_OK;
}

uint8_t* at(void* base, uint64_t off) { return reinterpret_cast<uint8_t*>(base) + off; }

// Run the k-means protocol of one stage on every problem of the batch.
// With the incremental buffers set (bf16 tokens, grouped heads), the first
// update of the stage also records the exact sums, counts, magnitude range and
// labels; each later update takes the heads that pass the exactness
// certificate incrementally (the moved tokens only) and the others in full.
int run_kmeans(const qkv_config* cfg, const KmBatch& b0, hipStream_t s) {
  KmBatch b = b0;
  const bool grouped = b.it[0].grp_off != nullptr;
  const bool inc = grouped && b.dtype == 1 && b.it[0].dsum != nullptr && cfg->kmeans_iters > 1;
  QKV_HIP(launch_kmeans_init(b, s));             // also clears emag and the close-call count
  for (int it = 0; it < cfg->kmeans_iters; ++it) {
    b.inc = inc ? (it == 0 ? 1 : 2) : 0;
    b.iter = it;
    QKV_HIP(launch_kmeans_assign(b, s));
    if (grouped) QKV_HIP(launch_kmeans_group(b, s));
    QKV_HIP(launch_kmeans_update(b, s));
    if (b.inc == 1) QKV_HIP(launch_kmeans_cert(b, s));
    if (b.inc == 2) QKV_HIP(launch_kmeans_update_delta(b, s));
  }
  return QKV_OK;
}

// The write path of qkv_quantize_chunk(s): problems share n_heads,
// n_clusters, kmeans_iters, n_stages, flags, n_tokens and dtype; each has its
// own slice of the workspace.
int quantize_batch(int32_t n, const qkv_config* const* cfgs, const qkv_tensor* const* xs,
                   const qkv_side* const* sides, void* const* packed, void* workspace, size_t workspace_bytes,
                   void* stream, const char* fn) {
  if (n < 1 || n > kKmMaxBatch) return fail(QKV_EINVAL, "%s: %d problems (1 to %d)", fn, n, kKmMaxBatch);
  if (!cfgs || !xs || !packed) return fail(QKV_EINVAL, "%s: NULL array", fn);
  const qkv_config* c0 = cfgs[0];
  QKV_TRY(check_config(c0, fn));
  QKV_TRY(check_tensor(xs[0], c0->n_heads, fn));
  const int64_t N = xs[0]->n_tokens;
  if (N < c0->n_clusters) return fail(QKV_EINVAL, "%s: n_tokens %lld < n_clusters %d", fn, (long long)N, c0->n_clusters);
  for (int p = 0; p < n; ++p) {
    const qkv_config* cfg = cfgs[p];
    QKV_TRY(check_config(cfg, fn));
    QKV_TRY(check_tensor(xs[p], c0->n_heads, fn));
    if (cfg->n_heads != c0->n_heads || cfg->n_clusters != c0->n_clusters || cfg->kmeans_iters != c0->kmeans_iters ||
        cfg->n_stages != c0->n_stages || cfg->flags != c0->flags)
      return fail(QKV_EINVAL, "%s: problem %d: configs of a batch must share n_heads, n_clusters, kmeans_iters, "
                  "n_stages and flags", fn, p);
    if (xs[p]->n_tokens != N || xs[p]->dtype != xs[0]->dtype)
      return fail(QKV_EINVAL, "%s: problem %d: tensors of a batch must share n_tokens and dtype", fn, p);
    if (!packed[p] || !aligned16(packed[p])) return fail(QKV_EINVAL, "%s: packed[%d] is NULL or not 16-byte aligned", fn, p);
    const qkv_side* side = sides ? sides[p] : nullptr;
    if (cfg->use_qsac && !(side && side->w)) return fail(QKV_EINVAL, "%s: problem %d: use_qsac needs side->w", fn, p);
    if (cfg->n_int4_channels > 0 && !(side && side->perm))
      return fail(QKV_EINVAL, "%s: problem %d: the mixed layout needs side->perm", fn, p);
    if (cfg->psac_rank > 0 && !(side && side->U)) return fail(QKV_EINVAL, "%s: problem %d: psac_rank > 0 needs side->U", fn, p);
  }
  const QuantWs ws = quant_ws(c0, N);
  const uint64_t per = align256(ws.bytes);
  QKV_TRY(check_ws(workspace, workspace_bytes, per * n, fn));

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int H = c0->n_heads;
  std::vector<qkv_layout> L(n);
  std::vector<ChunkDecode> g(n);
  std::vector<TensorView> y(n);
  KmBatch b{};
  b.n = n;
  b.dtype = xs[0]->dtype == QKV_F32 ? 0 : 1;
  b.H = H;
  b.C = c0->n_clusters;
  b.N = N;
  for (int p = 0; p < n; ++p) {
    layout_of(cfgs[p], N, &L[p]);
    g[p] = decode_of(cfgs[p], N, nullptr);
    y[p] = view_of(xs[p]);
    uint8_t* wsp = at(workspace, per * p);
    const qkv_side* side = sides ? sides[p] : nullptr;
    KmItem& it = b.it[p];
    it.w = cfgs[p]->use_qsac ? side->w : nullptr;
    it.c = reinterpret_cast<float*>(wsp + ws.c);
    it.amb_count = reinterpret_cast<int*>(wsp + ws.amb_count);
    it.counts = nullptr;
    const bool grouped = N <= kGroupMaxTokens;   // the update reads the tokens grouped by cluster
    it.grp_off = grouped ? reinterpret_cast<int*>(wsp + ws.grp_off) : nullptr;
    it.grp_list = grouped ? reinterpret_cast<uint16_t*>(wsp + ws.grp_list) : nullptr;
    it.ynorm = reinterpret_cast<float*>(wsp + ws.ynorm);
    // incremental updates: enabled per stage below (bf16 stage inputs only)
    it.dsum = grouped ? reinterpret_cast<double*>(wsp + ws.dsum) : nullptr;
    it.dcnt = grouped ? reinterpret_cast<int32_t*>(wsp + ws.dcnt) : nullptr;
    it.emag = grouped ? reinterpret_cast<uint32_t*>(wsp + ws.emag) : nullptr;
    it.cert = grouped ? reinterpret_cast<uint32_t*>(wsp + ws.cert) : nullptr;
    it.hlist = grouped ? reinterpret_cast<uint32_t*>(wsp + ws.hlist) : nullptr;
    it.prev = grouped ? wsp + ws.prev : nullptr;
  }
  for (int l = 0; l < c0->n_stages; ++l) {
    for (int p = 0; p < n; ++p) {
      uint8_t* base = reinterpret_cast<uint8_t*>(packed[p]);
      KmItem& it = b.it[p];
      it.y = y[p].ptr;
      it.stride_token = y[p].stride_token;
      it.stride_head = y[p].stride_head;
      it.labels = base + L[p].off_labels + (uint64_t)l * L[p].stage_bytes_labels;
      it.cent_bf16 = reinterpret_cast<uint16_t*>(base + L[p].off_centroids + (uint64_t)l * L[p].stage_bytes_centroids);
    }
    b.dtype = y[0].dtype;
    {
      // QSAC with the range factor: this stage's weights from its input
      RangeBatch rb{};
      rb.dtype = y[0].dtype;
      rb.H = H;
      rb.N = N;
      for (int p = 0; p < n; ++p) {
        if (cfgs[p]->use_qsac != 2) continue;
        uint8_t* wsp = at(workspace, per * p);
        const int r = rb.n++;
        rb.y[r] = y[p].ptr;
        rb.stride_token[r] = y[p].stride_token;
        rb.stride_head[r] = y[p].stride_head;
        rb.wq[r] = sides[p]->w;
        rb.w_out[r] = reinterpret_cast<float*>(wsp + ws.wq);
        rb.part[r] = reinterpret_cast<float*>(wsp + ws.rpart);
        b.it[p].w = rb.w_out[r];
      }
      if (rb.n > 0 && !(c0->flags & QKV_FLAG_RTN)) QKV_HIP(launch_qsac_range(rb, s));
    }
    if (c0->flags & QKV_FLAG_RTN) {
      for (int p = 0; p < n; ++p) {
        QKV_HIP(launch_fill_zero_u32(b.it[p].labels, L[p].stage_bytes_labels / 4, s));
        QKV_HIP(launch_fill_zero_u32(b.it[p].cent_bf16, L[p].stage_bytes_centroids / 4, s));
      }
    } else {
      QKV_TRY(run_kmeans(c0, b, s));
      QKV_HIP(launch_centroid_bf16(b, s));
    }
    const bool more = l + 1 < c0->n_stages;
    PackBatch pb, mb;                            // uniform-layout and mixed-layout problems
    pb.n = 0;
    mb.n = 0;
    for (int p = 0; p < n; ++p) {
      const qkv_config* cfg = cfgs[p];
      uint8_t* base = reinterpret_cast<uint8_t*>(packed[p]);
      uint8_t* wsp = at(workspace, per * p);
      PackArgs pa{};
      pa.y = y[p];
      pa.H = H;
      pa.C = c0->n_clusters;
      pa.N = (int)N;
      pa.labels = b.it[p].labels;
      pa.centroids = b.it[p].cent_bf16;
      pa.perm = cfg->n_int4_channels > 0 ? sides[p]->perm : nullptr;
      pa.bits = cfg->bits;
      pa.group = cfg->group;
      pa.n_int4 = cfg->n_int4_channels;
      pa.int4_words = g[p].int4_words;
      pa.codes = reinterpret_cast<uint32_t*>(base + L[p].off_codes + (uint64_t)l * L[p].stage_bytes_codes);
      pa.scales = reinterpret_cast<uint16_t*>(base + L[p].off_scales + (uint64_t)l * L[p].stage_bytes_scales);
      pa.words = g[p].words;
      pa.groups = g[p].groups;
      float* ynext = more ? reinterpret_cast<float*>(wsp + ((l % 2 == 0) ? ws.ybuf0 : ws.ybuf1)) : nullptr;
      pa.y_next = ynext;
      // the chunk's channel order section, written once (with the first stage)
      pa.perm_out = l == 0 && cfg->n_int4_channels > 0 ? base + L[p].off_perm : nullptr;
      if (pb.n > 0 && quant_pack_batchable(pa, pb.a[0])) pb.a[pb.n++] = pa;   // joins the batched launch
      else if (pb.n == 0 && quant_pack_batchable(pa, pa)) pb.a[pb.n++] = pa;
      else if (mb.n > 0 && quant_pack_mixed_batchable(pa, mb.a[0])) mb.a[mb.n++] = pa;
      else if (mb.n == 0 && quant_pack_mixed_batchable(pa, pa)) mb.a[mb.n++] = pa;
      else QKV_HIP(launch_quant_pack(pa, s));
      if (more) {
        // y_next is laid out [H][N][128]: token stride 128, head stride N*128
        y[p].ptr = ynext;
        y[p].dtype = 0;
        y[p].stride_token = kHeadDim;
        y[p].stride_head = N * kHeadDim;
      }
    }
    if (pb.n > 0) QKV_HIP(launch_quant_pack_batch(pb, s));
    if (mb.n > 0) QKV_HIP(launch_quant_pack_mixed_batch(mb, s));
  }
  for (int p = 0; p < n; ++p) {
    if (cfgs[p]->psac_rank > 0) {
      const ChunkDecode d = decode_of(cfgs[p], N, packed[p]);
      QKV_HIP(launch_psac_encode(d, view_of(xs[p]), sides[p]->U,
                                 reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(packed[p]) + L[p].off_psac), s));
    }
  }
  return ok();
}

}  // namespace

extern "C" {

int qkv_version(void) { return QKV_VERSION; }

const char* qkv_last_error(void) { return g_err.c_str(); }

int qkv_chunk_layout(const qkv_config* cfg, int64_t n_tokens, qkv_layout* out) {
  QKV_TRY(check_config(cfg, "qkv_chunk_layout"));
  if (!out) return fail(QKV_EINVAL, "qkv_chunk_layout: out is NULL");
  if (n_tokens < cfg->n_clusters || n_tokens > ((int64_t)1 << 24))
    return fail(QKV_EINVAL, "qkv_chunk_layout: n_tokens %lld must be in [n_clusters, 2^24]", (long long)n_tokens);
  layout_of(cfg, n_tokens, out);
  return ok();
}

int qkv_workspace_bytes(const qkv_config* cfg, int64_t max_chunk_tokens, int64_t n_query, int32_t n_chunks,
                        size_t* out) {
  QKV_TRY(check_config(cfg, "qkv_workspace_bytes"));
  if (!out) return fail(QKV_EINVAL, "qkv_workspace_bytes: out is NULL");
  if (max_chunk_tokens < 0 || n_query < 0 || n_chunks < 0 || n_chunks > kMaxChunks)
    return fail(QKV_EINVAL, "qkv_workspace_bytes: negative size or n_chunks > %d", kMaxChunks);
  uint64_t need = 0;
  if (max_chunk_tokens > 0) need = std::max(need, quant_ws(cfg, max_chunk_tokens).bytes);
  if (n_query > 0) {
    // mixed keys may take the mix4 path: room for their repacked codes
    const uint64_t krep = cfg->n_int4_channels > 0
                              ? (uint64_t)n_chunks * cfg->n_heads * (uint64_t)std::max<int64_t>(max_chunk_tokens, 1) * 64
                              : 0;
    // caches on the generic decode (several stages, INT4, groups not a multiple of 32): room for
    // their dense fp16 K and V rows
    const bool generic = cfg->n_stages > 1 || cfg->bits == 4 || cfg->group % 32 != 0;
    const uint64_t dense = generic ? 2ull * n_chunks * (uint64_t)std::max<int64_t>(max_chunk_tokens, 1) *
                                         cfg->n_heads * kHeadDim * 2
                                   : 0;
    // tiles for one more chunk: the fresh chunk of qkv_attend_fresh
    need = std::max(need, attend_ws(cfg->n_heads, n_query, n_chunks, max_tiles(std::max<int64_t>(max_chunk_tokens, 1), n_chunks + 1),
                                    max_split_rows(cfg->n_heads, n_query), kMaxClusters, kMaxClusters, krep, dense).bytes);
  }
  if (n_query > 0) need = std::max(need, psac_ws(cfg->n_heads));
  *out = (size_t)need;
  return ok();
}

int qkv_quantize_chunk(const qkv_config* cfg, const qkv_tensor* x, const qkv_side* side, void* packed,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_batch(1, &cfg, &x, &side, &packed, workspace, workspace_bytes, stream, "qkv_quantize_chunk");
}

int qkv_quantize_chunks(int32_t n, const qkv_config* const* cfgs, const qkv_tensor* const* xs,
                        const qkv_side* const* sides, void* const* packed, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return quantize_batch(n, cfgs, xs, sides, packed, workspace, workspace_bytes, stream, "qkv_quantize_chunks");
}

int qkv_quantize_chunk_noalloc(const qkv_config* cfg, const qkv_tensor* x, const qkv_side* side, void* packed,
                               void* stream) {
  const char* fn = "qkv_quantize_chunk_noalloc";
  QKV_TRY(check_config(cfg, fn));
  QKV_TRY(check_tensor(x, cfg->n_heads, fn));
  if (x->n_tokens < cfg->n_clusters)
    return fail(QKV_EINVAL, "%s: n_tokens %lld < n_clusters %d", fn, (long long)x->n_tokens, cfg->n_clusters);
  const uint64_t need = align256(quant_ws(cfg, x->n_tokens).bytes);
  if (need > kScratchBytes)
    return fail(QKV_EWORKSPACE, "%s: this chunk needs %llu bytes of scratch, the library holds %llu per device "
                "(use qkv_quantize_chunk with a workspace)", fn, (unsigned long long)need,
                (unsigned long long)kScratchBytes);
  void* scratch = nullptr;
  QKV_HIP(scratch_of_current_device(&scratch));
  return quantize_batch(1, &cfg, &x, &side, &packed, scratch, (size_t)kScratchBytes, stream, fn);
}

int qkv_quantize_chunks_workspace_bytes(const qkv_config* cfg, int64_t n_tokens, int32_t n, size_t* out) {
  QKV_TRY(check_config(cfg, "qkv_quantize_chunks_workspace_bytes"));
  if (!out) return fail(QKV_EINVAL, "qkv_quantize_chunks_workspace_bytes: out is NULL");
  if (n < 1 || n > kKmMaxBatch || n_tokens < cfg->n_clusters || n_tokens > ((int64_t)1 << 24))
    return fail(QKV_EINVAL, "qkv_quantize_chunks_workspace_bytes: n %d not in [1, %d] or n_tokens %lld out of range",
                n, kKmMaxBatch, (long long)n_tokens);
  *out = (size_t)(align256(quant_ws(cfg, n_tokens).bytes) * (uint64_t)n);
  return ok();
}

int qkv_dequantize(const qkv_config* cfg, int64_t n_tokens, const void* packed, const qkv_tensor* out, void* stream) {
  const char* fn = "qkv_dequantize";
  QKV_TRY(check_config(cfg, fn));
  if (n_tokens < cfg->n_clusters || n_tokens > ((int64_t)1 << 24))
    return fail(QKV_EINVAL, "%s: n_tokens %lld out of range", fn, (long long)n_tokens);
  if (!packed || !aligned16(packed)) return fail(QKV_EINVAL, "%s: packed is NULL or misaligned", fn);
  QKV_TRY(check_tensor(out, cfg->n_heads, fn));
  if (out->n_tokens != n_tokens) return fail(QKV_EINVAL, "%s: out has %lld tokens, chunk has %lld", fn,
                                             (long long)out->n_tokens, (long long)n_tokens);
  const ChunkDecode d = decode_of(cfg, n_tokens, packed);
  QKV_HIP(launch_dequantize(d, out->ptr, out->dtype == QKV_F32 ? 0 : 1, out->stride_token, out->stride_head,
                            reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

namespace {

// qkv_attend and qkv_attend_fresh: kf/vf (may be NULL) is a fresh chunk whose
// keys follow the packed chunks, seen by query i up to frame i / frame_tokens.
int attend_impl(const char* fn, const qkv_config* k_cfg, const qkv_config* v_cfg, const qkv_tensor* q,
                const void* const* k_chunks, const void* const* v_chunks, const int64_t* chunk_tokens,
                int32_t n_chunks, const qkv_tensor* kf, const qkv_tensor* vf, int32_t frame_tokens, const float* U,
                int32_t causal, float softmax_scale, const qkv_tensor* out, float* logits_debug, void* workspace,
                size_t workspace_bytes, void* stream) {
  QKV_TRY(check_config(k_cfg, fn));
  QKV_TRY(check_config(v_cfg, fn));
  if (k_cfg->n_heads != v_cfg->n_heads) return fail(QKV_EINVAL, "%s: K and V head counts differ", fn);
  if (v_cfg->psac_rank != 0) return fail(QKV_EINVAL, "%s: PSAC applies to keys only (v_cfg->psac_rank != 0)", fn);
  const int H = k_cfg->n_heads;
  QKV_TRY(check_tensor(q, H, fn));
  QKV_TRY(check_tensor(out, H, fn));
  if (out->dtype != QKV_F32) return fail(QKV_EINVAL, "%s: out must be f32", fn);
  if (out->n_tokens != q->n_tokens) return fail(QKV_EINVAL, "%s: out and q token counts differ", fn);
  const bool fresh = kf != nullptr;
  if (n_chunks < (fresh ? 0 : 1) || n_chunks > kMaxChunks)
    return fail(QKV_EINVAL, "%s: n_chunks %d not in [%d, %d]", fn, n_chunks, fresh ? 0 : 1, kMaxChunks);
  if (n_chunks > 0 && (!k_chunks || !v_chunks || !chunk_tokens)) return fail(QKV_EINVAL, "%s: chunk arrays are NULL", fn);
  int64_t n_fresh = 0;
  if (fresh) {
    QKV_TRY(check_tensor(kf, H, fn));
    QKV_TRY(check_tensor(vf, H, fn));
    n_fresh = kf->n_tokens;
    if (vf->n_tokens != n_fresh) return fail(QKV_EINVAL, "%s: fresh keys and values hold different token counts", fn);
    if (q->n_tokens != n_fresh)
      return fail(QKV_EINVAL, "%s: the queries must be the fresh chunk's %lld tokens (got %lld)", fn, (long long)n_fresh,
                  (long long)q->n_tokens);
    if (frame_tokens < 1) return fail(QKV_EINVAL, "%s: frame_tokens %d must be >= 1", fn, frame_tokens);
    if (q->dtype != QKV_BF16) return fail(QKV_EUNSUPPORTED, "%s: a fresh chunk needs bf16 queries", fn);
    if (n_fresh > ((int64_t)1 << 24)) return fail(QKV_EINVAL, "%s: fresh chunk of %lld tokens", fn, (long long)n_fresh);
  }
  if (k_cfg->psac_rank > 0 && !U) return fail(QKV_EINVAL, "%s: k_cfg->psac_rank > 0 needs U", fn);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f) return fail(QKV_EINVAL, "%s: softmax_scale must be >= 0", fn);
  const int64_t Nq = q->n_tokens;
  std::vector<ChunkRec> recs(n_chunks);
  int64_t Nk = 0, n_tiles = 0;
  for (int i = 0; i < n_chunks; ++i) {
    const int64_t n = chunk_tokens[i];
    if (n < std::max(k_cfg->n_clusters, v_cfg->n_clusters) || n > ((int64_t)1 << 24))
      return fail(QKV_EINVAL, "%s: chunk %d has %lld tokens", fn, i, (long long)n);
    if (!k_chunks[i] || !v_chunks[i] || !aligned16(k_chunks[i]) || !aligned16(v_chunks[i]))
      return fail(QKV_EINVAL, "%s: chunk %d pointer NULL or misaligned", fn, i);
    const ChunkDecode dk = make_decode(params_of(k_cfg), n, k_chunks[i]);
    const ChunkDecode dv = make_decode(params_of(v_cfg), n, v_chunks[i]);
    recs[i].kbase = dk.base;
    recs[i].vbase = dv.base;
    recs[i].kcodes = dk.base + dk.off_codes;
    recs[i].kscales = dk.base + dk.off_scales;
    recs[i].klabels = dk.base + dk.off_labels;
    recs[i].kcent = dk.base + dk.off_centroids;
    recs[i].kpsac = dk.base + dk.off_psac;
    recs[i].vcodes = dv.base + dv.off_codes;
    recs[i].vscales = dv.base + dv.off_scales;
    recs[i].vlabels = dv.base + dv.off_labels;
    recs[i].vcent = dv.base + dv.off_centroids;
    recs[i].token_start = Nk;
    recs[i].n = (int32_t)n;
    recs[i].tile_start = (int32_t)n_tiles;
    Nk += n;
    n_tiles += (n + kTileKeys - 1) / kTileKeys;
  }
  const int64_t Nk_cache = Nk, n_cache_tiles = n_tiles;
  Nk += n_fresh;
  n_tiles += (n_fresh + kTileKeys - 1) / kTileKeys;
  if (Nk > ((int64_t)1 << 31) - 1) return fail(QKV_EINVAL, "%s: the cache holds more than 2^31 tokens", fn);
  if (causal && !fresh && Nk != Nq) return fail(QKV_EINVAL, "%s: causal attention needs as many queries as cached keys", fn);
  // A workspace sized by qkv_workspace_bytes for at least these queries and
  // chunks always suffices: ns <= split_cap(H, Nq).
  const int ns = choose_splits(H, Nq, n_tiles);
  auto fast = [](const qkv_config* c) {
    return c->n_stages == 1 && c->n_int4_channels == 0 && c->bits == 2 && c->group % 32 == 0;
  };
  const bool kfast = fast(k_cfg), vfast = fast(v_cfg);
  // mixed INT4/INT2 keys of one stage: the mix4 path when their groups allow it
  MixOrder mix{};
  const bool kmix = !kfast && k_cfg->n_stages == 1 && k_cfg->n_int4_channels > 0 && k_cfg->psac_rank == 0 &&
                    q->dtype == QKV_BF16 && mix4_order(params_of(k_cfg), &mix);
  const int kmode = kfast ? 1 : kmix ? 2 : 0;
  const int kC16 = kmode ? k_cfg->n_clusters : 0, vC16 = vfast ? v_cfg->n_clusters : 0;
  // A fresh chunk over packed chunks with the lean decode (fast K and V, bf16 queries, no PSAC, no
  // logits): the cached tiles take the lean kernel variant in a launch of their own -- non-causal, as
  // every cached key is visible to every query of the fresh chunk -- and the fresh chunk's tiles the
  // fresh-chunk variant in a second one; the merge joins their partial rows (at most split_cap rows
  // per query in all, as the workspace provides).
  const int cap = split_cap(H, Nq);
  const bool two = fresh && n_chunks > 0 && kmode != 0 && vfast && q->dtype == QKV_BF16 && k_cfg->psac_rank == 0 &&
                   !logits_debug && cap >= 2;
  // A cache on the generic decode (bf16 queries, no PSAC), when the workspace has room:
  // decoded once into dense fp16 rows (k_dense_decode, the tile decode's own arithmetic and scaling),
  // then attended as the tiles of one fresh chunk, so the tile loop does no per-element decode.
  const int64_t n_dtiles = (Nk + kTileKeys - 1) / kTileKeys;
  bool dense = false;
  if (!fresh && n_chunks > 0 && (kmode == 0 || !vfast) && q->dtype == QKV_BF16 && k_cfg->psac_rank == 0) {
    const int nsd = choose_splits(H, Nq, n_dtiles);
    dense = workspace_bytes >= attend_ws(H, Nq, n_chunks, std::max<int64_t>(n_tiles, n_dtiles), nsd > 1 ? (int64_t)nsd * Nq : 0,
                                         0, 0, 0, 2ull * Nk * H * kHeadDim * 2).bytes;
  }
  const int ns_cache = two ? std::min(choose_splits(H, Nq, n_cache_tiles), cap - 1) : 0;
  const int ns_total = two ? ns_cache + 1 : ns;
  const int ns_dense = dense ? choose_splits(H, Nq, n_dtiles) : 0;
  const AttendWs ws = dense ? attend_ws(H, Nq, n_chunks, std::max<int64_t>(n_tiles, n_dtiles),
                                        ns_dense > 1 ? (int64_t)ns_dense * Nq : 0, 0, 0, 0, 2ull * Nk * H * kHeadDim * 2)
                            : attend_ws(H, Nq, n_chunks, n_tiles, ns_total > 1 ? (int64_t)ns_total * Nq : 0, kC16, vC16,
                                        kmix ? (uint64_t)H * Nk * 64 : 0);
  QKV_TRY(check_ws(workspace, workspace_bytes, ws.bytes, fn));
  if (kmix && !dense) {
    uint64_t off = 0;
    for (int i = 0; i < n_chunks; ++i) {
      recs[i].krep = at(workspace, ws.krep + off);
      off += (uint64_t)H * recs[i].n * 64;
    }
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ChunkRec* drecs = reinterpret_cast<ChunkRec*>(at(workspace, ws.chunks));
  uint32_t* range = reinterpret_cast<uint32_t*>(at(workspace, ws.range));
  for (int first = 0; first < n_chunks; first += kChunkBatch) {
    ChunkBatch b;
    std::memset(&b, 0, sizeof b);
    b.first = first;
    b.count = std::min(kChunkBatch, n_chunks - first);
    for (int i = 0; i < b.count; ++i) b.rec[i] = recs[first + i];
    QKV_HIP(launch_upload_chunks(b, drecs, range, mix, kmix ? reinterpret_cast<MixOrder*>(at(workspace, ws.mix)) : nullptr,
                                 s));
  }
  if (n_chunks == 0) {                           // a fresh chunk alone: the upload still clears the range record
    ChunkBatch b;
    std::memset(&b, 0, sizeof b);
    QKV_HIP(launch_upload_chunks(b, drecs, range, mix, nullptr, s));
  }
  const MixOrder* dmix = kmix ? reinterpret_cast<const MixOrder*>(at(workspace, ws.mix)) : nullptr;
  int64_t max_n = 0;
  for (int i = 0; i < n_chunks; ++i) max_n = std::max<int64_t>(max_n, recs[i].n);
  if (kmix && !dense) QKV_HIP(launch_repack_mix(drecs, n_chunks, (int)max_n, params_of(k_cfg), dmix, s));
  // operand range of the fp16 MFMAs: largest stored scale, centroid, PSAC
  // coefficient and query (the kernels below derive their power-of-two scaling from it)
  TensorView kfv{}, vfv{};
  if (fresh) {
    kfv = view_of(kf);
    vfv = view_of(vf);
  }
  QKV_HIP(launch_range_scan(drecs, n_chunks, params_of(k_cfg), params_of(v_cfg), view_of(q), (int)Nq, kfv, vfv,
                            (int)n_fresh, range, s));
  TileRec* dtiles = reinterpret_cast<TileRec*>(at(workspace, ws.tiles));
  if (dense) {
    uint16_t* dk = reinterpret_cast<uint16_t*>(at(workspace, ws.dense));
    uint16_t* dv = dk + (size_t)Nk * H * kHeadDim;
    QKV_HIP(launch_dense_decode(drecs, n_chunks, (int)max_n, H, params_of(k_cfg), params_of(v_cfg), range, dk, dv, s));
    const TokenBytes tb{0, 0, 0, 0, 0};
    QKV_HIP(launch_tile_table(drecs, 0, (int)n_dtiles, 0, (int)Nk, 0, tb, H, k_cfg->n_clusters, v_cfg->n_clusters, nullptr,
                              nullptr, dtiles, s));
    AttendArgs a{};
    a.q = view_of(q);
    a.H = H;
    a.Nq = (int)Nq;
    a.Nk = Nk;
    a.n_chunks = 0;
    a.n_tiles = (int)n_dtiles;
    a.kp = params_of(k_cfg);
    a.vp = params_of(v_cfg);
    a.chunks = drecs;
    a.tiles = dtiles;
    a.qu = reinterpret_cast<float*>(at(workspace, ws.qu));
    a.causal = causal ? 1 : 0;                   // token-causal: frames of one token from key 0
    a.mask_F = causal ? 1 : (1 << 30);
    a.mask_base = 0;
    a.kf = TensorView{dk, 2, Nk, (int64_t)H * kHeadDim, kHeadDim};
    a.vf = TensorView{dv, 2, Nk, (int64_t)H * kHeadDim, kHeadDim};
    a.n_cache_tiles = 0;
    a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)kHeadDim);
    a.n_split = ns_dense;
    a.tile_lo = 0;
    a.split_base = 0;
    a.n_split_total = ns_dense;
    a.part_o = reinterpret_cast<float*>(at(workspace, ws.part_o));
    a.part_ml = reinterpret_cast<float*>(at(workspace, ws.part_ml));
    a.out = reinterpret_cast<float*>(out->ptr);
    a.out_stride_token = out->stride_token;
    a.out_stride_head = out->stride_head;
    a.logits = logits_debug;                     // key index = the dense row = the cache's token index
    a.range = range;
    a.k_mode = 1;                                // the lean fresh-chunk variant: every tile is a dense one
    a.mixp = nullptr;
    a.v_uniform_int2_1stage = true;
    QKV_HIP(launch_attend(a, s));
    return ok();
  }
  uint16_t* k16 = kmode ? reinterpret_cast<uint16_t*>(at(workspace, ws.k16)) : nullptr;
  uint16_t* v16 = vfast ? reinterpret_cast<uint16_t*>(at(workspace, ws.v16)) : nullptr;
  QKV_HIP(launch_centroids_f16(drecs, n_chunks, params_of(k_cfg), params_of(v_cfg), range, dmix, k16, v16, s));
  {
    const ChunkDecode dk = make_decode(params_of(k_cfg), 1, nullptr), dv = make_decode(params_of(v_cfg), 1, nullptr);
    const TokenBytes tb{kmix ? 64 : dk.words * 4, dv.words * 4, dk.groups * 2, dv.groups * 2, k_cfg->psac_rank * 2};
    QKV_HIP(launch_tile_table(drecs, n_chunks, (int)n_tiles, (int)n_cache_tiles, (int)n_fresh, Nk_cache, tb, H,
                              k_cfg->n_clusters, v_cfg->n_clusters, k16, v16, dtiles, s));
  }

  AttendArgs a;
  a.q = view_of(q);
  a.H = H;
  a.Nq = (int)Nq;
  a.Nk = Nk;
  a.n_chunks = n_chunks;
  a.n_tiles = (int)n_tiles;
  a.kp = params_of(k_cfg);
  a.vp = params_of(v_cfg);
  a.chunks = drecs;
  a.tiles = dtiles;
  a.U = U;
  a.psac_rank = k_cfg->psac_rank;
  a.qu = reinterpret_cast<float*>(at(workspace, ws.qu));
  a.causal = (causal || fresh) ? 1 : 0;
  a.mask_F = fresh ? frame_tokens : 1;           // token-causal: key j visible to query i iff j < i + 1
  a.mask_base = fresh ? (int)Nk_cache : 0;
  a.kf = kfv;
  a.vf = vfv;
  a.n_cache_tiles = (int)n_cache_tiles;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)kHeadDim);
  a.n_split = ns;
  a.tile_lo = 0;
  a.split_base = 0;
  a.n_split_total = ns;
  a.part_o = reinterpret_cast<float*>(at(workspace, ws.part_o));
  a.part_ml = reinterpret_cast<float*>(at(workspace, ws.part_ml));
  a.out = reinterpret_cast<float*>(out->ptr);
  a.out_stride_token = out->stride_token;
  a.out_stride_head = out->stride_head;
  a.logits = logits_debug;
  a.range = range;
  a.k_mode = kmode;
  a.mixp = dmix;
  a.v_uniform_int2_1stage = vfast;
  if (two) {
    AttendArgs c = a;                            // the cached tiles
    c.kf = TensorView{};
    c.vf = TensorView{};
    c.causal = 0;
    c.mask_F = 1;
    c.mask_base = 0;
    c.n_tiles = (int)n_cache_tiles;
    c.n_split = ns_cache;
    c.n_split_total = ns_total;
    QKV_HIP(launch_attend(c, s));
    a.tile_lo = (int)n_cache_tiles;              // the fresh chunk's tiles, then the merge
    a.n_split = 1;
    a.split_base = ns_cache;
    a.n_split_total = ns_total;
  }
  QKV_HIP(launch_attend(a, s));
  return ok();
}

}  // namespace

extern "C" {

int qkv_attend(const qkv_config* k_cfg, const qkv_config* v_cfg, const qkv_tensor* q, const void* const* k_chunks,
               const void* const* v_chunks, const int64_t* chunk_tokens, int32_t n_chunks, const float* U,
               int32_t causal, float softmax_scale, const qkv_tensor* out, float* logits_debug, void* workspace,
               size_t workspace_bytes, void* stream) {
  return attend_impl("qkv_attend", k_cfg, v_cfg, q, k_chunks, v_chunks, chunk_tokens, n_chunks, nullptr, nullptr, 0, U,
                     causal, softmax_scale, out, logits_debug, workspace, workspace_bytes, stream);
}

int qkv_attend_fresh(const qkv_config* k_cfg, const qkv_config* v_cfg, const qkv_tensor* q,
                     const void* const* k_chunks, const void* const* v_chunks, const int64_t* chunk_tokens,
                     int32_t n_chunks, const qkv_tensor* k_fresh, const qkv_tensor* v_fresh, int32_t frame_tokens,
                     const float* U, float softmax_scale, const qkv_tensor* out, float* logits_debug,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_fresh || !v_fresh) return fail(QKV_EINVAL, "qkv_attend_fresh: k_fresh or v_fresh is NULL");
  return attend_impl("qkv_attend_fresh", k_cfg, v_cfg, q, k_chunks, v_chunks, chunk_tokens, n_chunks, k_fresh, v_fresh,
                     frame_tokens, U, 1, softmax_scale, out, logits_debug, workspace, workspace_bytes, stream);
}

int qkv_psac_fit(const qkv_tensor* q_hist, int32_t n_heads, int32_t rank, int32_t n_int4, float* U_out, float* w_out, uint8_t* perm_out,
                 float* energy_out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "qkv_psac_fit";
  if (!q_hist) return fail(QKV_EINVAL, "%s: q_hist is NULL", fn);
  if (rank < 0 || rank > kMaxRank) return fail(QKV_EINVAL, "%s: rank %d not in [0, 8]", fn, rank);
  if (n_int4 < 0 || n_int4 >= kHeadDim) return fail(QKV_EINVAL, "%s: n_int4 %d not in [0, 127]", fn, n_int4);
  if (rank > 0 && !U_out) return fail(QKV_EINVAL, "%s: rank > 0 needs U_out", fn);
  const int H = n_heads;
  if (H < 1 || H > 1024) return fail(QKV_EINVAL, "%s: n_heads %d not in [1, 1024]", fn, H);
  QKV_TRY(check_tensor(q_hist, H, fn));
  QKV_TRY(check_ws(workspace, workspace_bytes, psac_ws(H), fn));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  double* partial = reinterpret_cast<double*>(workspace);
  double* m = reinterpret_cast<double*>(at(workspace, align256((uint64_t)kGramSplit * H * kHeadDim * kHeadDim * 8)));
  // the eigendecomposition needs all of M; the activity and the channel order only its diagonal
  const bool full = rank > 0 || energy_out;
  std::vector<double> hd((size_t)H * kHeadDim);
  std::vector<float> energy(H);
  if (full) {
    // the partials are consumed by the reduction: they then hold M's diagonal, the energies
    // and the solver's rotation record (room for 16 sweeps per head)
    double* dg = partial;
    float* en = reinterpret_cast<float*>(dg + (size_t)H * kHeadDim);
    const uint64_t rot_off = align256((uint64_t)H * kHeadDim * 8 + (uint64_t)H * 4);
    const uint64_t part_bytes = (uint64_t)kGramSplit * H * kHeadDim * kHeadDim * 8;
    QKV_HIP(launch_gram(view_of(q_hist), H, partial, kGramSplit, m, s));
    QKV_HIP(launch_eigh(m, H, at(workspace, rot_off), part_bytes - rot_off, rank, rank > 0 ? U_out : nullptr, en, dg, s));
    QKV_HIP(hipMemcpyAsync(hd.data(), dg, hd.size() * 8, hipMemcpyDeviceToHost, s));
    QKV_HIP(hipMemcpyAsync(energy.data(), en, energy.size() * 4, hipMemcpyDeviceToHost, s));
  } else {
    QKV_HIP(launch_gram_diag(view_of(q_hist), H, partial, kGramSplit, m, s));
    QKV_HIP(hipMemcpyAsync(hd.data(), m, hd.size() * 8, hipMemcpyDeviceToHost, s));
  }
  QKV_HIP(hipStreamSynchronize(s));

  const double n = (double)q_hist->n_tokens;
  std::vector<float> hw((size_t)H * kHeadDim);
  std::vector<uint8_t> hperm((size_t)H * kHeadDim);
  for (int h = 0; h < H; ++h)
    for (int k = 0; k < kHeadDim; ++k) hw[(size_t)h * kHeadDim + k] = (float)(hd[(size_t)h * kHeadDim + k] / n);
  for (int h = 0; h < H; ++h) {
    std::vector<int> order(kHeadDim);
    for (int k = 0; k < kHeadDim; ++k) order[k] = k;
    const float* wh = hw.data() + (size_t)h * kHeadDim;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return wh[x] > wh[y]; });
    std::vector<int> top(order.begin(), order.begin() + n_int4), rest(order.begin() + n_int4, order.end());
    std::sort(top.begin(), top.end());
    std::sort(rest.begin(), rest.end());
    int p = 0;
    for (int k : top) hperm[(size_t)h * kHeadDim + p++] = (uint8_t)k;
    for (int k : rest) hperm[(size_t)h * kHeadDim + p++] = (uint8_t)k;
  }
  // outputs on the caller's stream, complete (host buffers released) before the return
  if (w_out) QKV_HIP(hipMemcpyAsync(w_out, hw.data(), hw.size() * 4, hipMemcpyHostToDevice, s));
  if (perm_out && n_int4 > 0) QKV_HIP(hipMemcpyAsync(perm_out, hperm.data(), hperm.size(), hipMemcpyHostToDevice, s));
  QKV_HIP(hipStreamSynchronize(s));
  if (energy_out) std::memcpy(energy_out, energy.data(), H * sizeof(float));
  return ok();
}

// A one-problem k-means batch over caller buffers (step-level entry points).
KmBatch single_batch(const qkv_config* cfg, const qkv_tensor* y, const float* w, float* centroids, uint8_t* labels,
                     int32_t* counts, void* workspace, const QuantWs& ws) {
  KmBatch b{};
  b.n = 1;
  b.dtype = y->dtype == QKV_F32 ? 0 : 1;
  b.H = cfg->n_heads;
  b.C = cfg->n_clusters;
  b.N = y->n_tokens;
  const TensorView v = view_of(y);
  KmItem& it = b.it[0];
  it.y = v.ptr;
  it.stride_token = v.stride_token;
  it.stride_head = v.stride_head;
  it.w = w;
  it.c = centroids;
  it.labels = labels;
  it.amb_count = reinterpret_cast<int*>(at(workspace, ws.amb_count));
  it.counts = counts;
  it.cent_bf16 = nullptr;
  it.grp_off = nullptr;
  it.grp_list = nullptr;
  return b;
}

int qkv_kmeans_assign(const qkv_config* cfg, const qkv_tensor* y, const float* centroids, const float* w,
                      uint8_t* labels, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "qkv_kmeans_assign";
  QKV_TRY(check_config(cfg, fn));
  QKV_TRY(check_tensor(y, cfg->n_heads, fn));
  if (!centroids || !labels) return fail(QKV_EINVAL, "%s: centroids/labels NULL", fn);
  if (y->n_tokens < cfg->n_clusters) return fail(QKV_EINVAL, "%s: n_tokens < n_clusters", fn);
  const QuantWs ws = quant_ws(cfg, y->n_tokens);
  QKV_TRY(check_ws(workspace, workspace_bytes, ws.ybuf0, fn));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the kernels only read the centroids here
  const KmBatch b = single_batch(cfg, y, w, const_cast<float*>(centroids), labels, nullptr, workspace, ws);
  QKV_HIP(launch_fill_zero_u32(b.it[0].amb_count, 1, s));   // the close-call count (statistics)
  QKV_HIP(launch_kmeans_assign(b, s));
  return ok();
}

int qkv_kmeans_update(const qkv_config* cfg, const qkv_tensor* y, const uint8_t* labels, float* centroids,
                      int32_t* counts, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "qkv_kmeans_update";
  QKV_TRY(check_config(cfg, fn));
  QKV_TRY(check_tensor(y, cfg->n_heads, fn));
  if (!centroids || !labels) return fail(QKV_EINVAL, "%s: centroids/labels NULL", fn);
  const QuantWs ws = quant_ws(cfg, y->n_tokens);
  QKV_TRY(check_ws(workspace, workspace_bytes, ws.ybuf0, fn));
  const KmBatch b = single_batch(cfg, y, nullptr, centroids, const_cast<uint8_t*>(labels), counts, workspace, ws);
  QKV_HIP(launch_kmeans_update(b, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

int qkv_quant_pack(const qkv_config* cfg, const qkv_tensor* y, const uint8_t* labels, const float* centroids,
                   const uint8_t* perm, void* packed, int32_t stage, float* y_next, void* stream) {
  const char* fn = "qkv_quant_pack";
  QKV_TRY(check_config(cfg, fn));
  QKV_TRY(check_tensor(y, cfg->n_heads, fn));
  if (!labels || !centroids || !packed || !aligned16(packed)) return fail(QKV_EINVAL, "%s: NULL or misaligned pointer", fn);
  if (stage < 0 || stage >= cfg->n_stages) return fail(QKV_EINVAL, "%s: stage %d not in [0, n_stages)", fn, stage);
  if (cfg->n_int4_channels > 0 && !perm) return fail(QKV_EINVAL, "%s: the mixed layout needs perm", fn);
  const int64_t N = y->n_tokens;
  if (N < cfg->n_clusters) return fail(QKV_EINVAL, "%s: n_tokens < n_clusters", fn);
  qkv_layout L;
  layout_of(cfg, N, &L);
  const ChunkDecode g = decode_of(cfg, N, nullptr);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = reinterpret_cast<uint8_t*>(packed);
  uint8_t* lab_dst = base + L.off_labels + (uint64_t)stage * L.stage_bytes_labels;
  if (lab_dst != labels) QKV_HIP(hipMemcpyAsync(lab_dst, labels, (size_t)cfg->n_heads * N, hipMemcpyDeviceToDevice, s));
  uint16_t* cent = reinterpret_cast<uint16_t*>(base + L.off_centroids + (uint64_t)stage * L.stage_bytes_centroids);
  {
    KmBatch b{};
    b.n = 1;
    b.H = cfg->n_heads;
    b.C = cfg->n_clusters;
    b.it[0].c = const_cast<float*>(centroids);   // read only
    b.it[0].cent_bf16 = cent;
    QKV_HIP(launch_centroid_bf16(b, s));
  }
  const uint8_t* pm = cfg->n_int4_channels > 0 ? perm : nullptr;
  if (pm) QKV_HIP(launch_copy_perm(pm, base + L.off_perm, cfg->n_heads, s));
  PackArgs pa{};
  pa.y = view_of(y);
  pa.H = cfg->n_heads;
  pa.C = cfg->n_clusters;
  pa.N = (int)N;
  pa.labels = lab_dst;
  pa.centroids = cent;
  pa.perm = pm;
  pa.bits = cfg->bits;
  pa.group = cfg->group;
  pa.n_int4 = cfg->n_int4_channels;
  pa.int4_words = g.int4_words;
  pa.codes = reinterpret_cast<uint32_t*>(base + L.off_codes + (uint64_t)stage * L.stage_bytes_codes);
  pa.scales = reinterpret_cast<uint16_t*>(base + L.off_scales + (uint64_t)stage * L.stage_bytes_scales);
  pa.words = g.words;
  pa.groups = g.groups;
  pa.y_next = y_next;
  QKV_HIP(launch_quant_pack(pa, s));
  return ok();
}

}  // extern "C"

namespace {

int check_tcfg(const qkv_tcfg* c, const char* what) {
  if (!c) return fail(QKV_EINVAL, "%s: cfg is NULL", what);
  if (c->n_heads < 1 || c->n_heads > 256) return fail(QKV_EINVAL, "%s: n_heads %d not in [1, 256]", what, c->n_heads);
  if (c->frame_tokens < 1 || c->frame_tokens > (1 << 24))
    return fail(QKV_EINVAL, "%s: frame_tokens %d not in [1, 2^24]", what, c->frame_tokens);
  if (c->bits != 2 && c->bits != 4) return fail(QKV_EINVAL, "%s: bits must be 2 or 4", what);
  if (c->anchor_every < 1) return fail(QKV_EINVAL, "%s: anchor_every must be >= 1", what);
  if (!(c->decay >= 0.0f && c->decay <= 1.0f)) return fail(QKV_EINVAL, "%s: decay must be in [0, 1]", what);
  return QKV_OK;
}

struct TLayout {
  uint64_t bytes;
  uint64_t frame_off[kTMaxFrames];
  uint64_t sec_codes, sec_lo, sec_scale, sec_oval, sec_oidx, coded_bytes, anchor_bytes;
};

TLayout temporal_layout(const qkv_tcfg* c, int64_t frame0, int n_frames) {
  const uint64_t th = (uint64_t)c->frame_tokens * c->n_heads;
  TLayout L;
  L.sec_codes = 0;
  L.sec_lo = align256(th * 4 * c->bits * 4);
  L.sec_scale = L.sec_lo + align256(th * 4 * 2);
  L.sec_oval = L.sec_scale + align256(th * 4 * 2);
  L.sec_oidx = L.sec_oval + align256(th * 4 * 2);
  L.coded_bytes = L.sec_oidx + align256(th * 4);
  L.anchor_bytes = align256(th * kHeadDim * 2);
  uint64_t off = 0;
  for (int f = 0; f < n_frames; ++f) {
    L.frame_off[f] = off;
    off += (frame0 + f) % c->anchor_every == 0 ? L.anchor_bytes : L.coded_bytes;
  }
  L.bytes = off;
  return L;
}

int check_trun(const qkv_tcfg* c, int64_t frame0, int32_t n_frames, const char* what) {
  QKV_TRY(check_tcfg(c, what));
  if (frame0 < 0) return fail(QKV_EINVAL, "%s: frame0 %lld < 0", what, (long long)frame0);
  if (n_frames < 1 || n_frames > kTMaxFrames) return fail(QKV_EINVAL, "%s: n_frames %d not in [1, %d]", what, n_frames, kTMaxFrames);
  return QKV_OK;
}

TCodecArgs tcodec_args(const qkv_tcfg* c, int64_t frame0, int32_t n_frames, const TLayout& L) {
  TCodecArgs a{};
  a.H = c->n_heads;
  a.P = c->frame_tokens;
  a.bits = c->bits;
  a.anchor_every = c->anchor_every;
  a.n_frames = n_frames;
  a.decay = c->decay;
  a.frame0 = frame0;
  int fa = -1;
  for (int f = 0; f < n_frames; ++f) {
    a.frame_off[f] = L.frame_off[f];
    if ((frame0 + f) % c->anchor_every == 0) fa = f;
    a.anc_frame[f] = (int8_t)fa;
  }
  a.sec_codes = L.sec_codes;
  a.sec_lo = L.sec_lo;
  a.sec_scale = L.sec_scale;
  a.sec_oval = L.sec_oval;
  a.sec_oidx = L.sec_oidx;
  return a;
}

}  // namespace

extern "C" {

int qkv_temporal_layout(const qkv_tcfg* cfg, int64_t frame0, int32_t n_frames, size_t* bytes, size_t* frame_offsets) {
  QKV_TRY(check_trun(cfg, frame0, n_frames, "qkv_temporal_layout"));
  if (!bytes) return fail(QKV_EINVAL, "qkv_temporal_layout: bytes is NULL");
  const TLayout L = temporal_layout(cfg, frame0, n_frames);
  *bytes = (size_t)L.bytes;
  if (frame_offsets)
    for (int f = 0; f < n_frames; ++f) frame_offsets[f] = (size_t)L.frame_off[f];
  return ok();
}

int qkv_temporal_state_bytes(const qkv_tcfg* cfg, size_t* bytes) {
  QKV_TRY(check_tcfg(cfg, "qkv_temporal_state_bytes"));
  if (!bytes) return fail(QKV_EINVAL, "qkv_temporal_state_bytes: bytes is NULL");
  *bytes = (size_t)cfg->frame_tokens * cfg->n_heads * kHeadDim * 6;
  return ok();
}

int qkv_temporal_encode(const qkv_tcfg* cfg, const qkv_tensor* x, int64_t frame0, void* state, void* packed,
                        void* stream) {
  const char* fn = "qkv_temporal_encode";
  QKV_TRY(check_tcfg(cfg, fn));
  QKV_TRY(check_tensor(x, cfg->n_heads, fn));
  if (x->n_tokens % cfg->frame_tokens) return fail(QKV_EINVAL, "%s: n_tokens %lld is not a whole number of frames of %d tokens",
                                                   fn, (long long)x->n_tokens, cfg->frame_tokens);
  const int64_t nf = x->n_tokens / cfg->frame_tokens;
  QKV_TRY(check_trun(cfg, frame0, (int32_t)std::min<int64_t>(nf, INT32_MAX), fn));
  if (!state || !aligned16(state)) return fail(QKV_EINVAL, "%s: state is NULL or not 16-byte aligned", fn);
  if (!packed || !aligned16(packed)) return fail(QKV_EINVAL, "%s: packed is NULL or not 16-byte aligned", fn);
  const TLayout L = temporal_layout(cfg, frame0, (int)nf);
  TCodecArgs a = tcodec_args(cfg, frame0, (int32_t)nf, L);
  a.x = view_of(x);
  a.fb = reinterpret_cast<float*>(state);
  a.anchor = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(state) + (uint64_t)cfg->frame_tokens * cfg->n_heads * kHeadDim * 4);
  a.packed = reinterpret_cast<uint8_t*>(packed);
  QKV_HIP(launch_temporal_encode(a, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

int qkv_temporal_decode(const qkv_tcfg* cfg, int64_t frame0, int32_t n_frames, const void* packed, const void* anchor,
                        const qkv_tensor* out, void* stream) {
  const char* fn = "qkv_temporal_decode";
  QKV_TRY(check_trun(cfg, frame0, n_frames, fn));
  QKV_TRY(check_tensor(out, cfg->n_heads, fn));
  if (out->n_tokens != (int64_t)n_frames * cfg->frame_tokens)
    return fail(QKV_EINVAL, "%s: out has %lld tokens, the run %lld", fn, (long long)out->n_tokens,
                (long long)n_frames * cfg->frame_tokens);
  if (!packed || !aligned16(packed)) return fail(QKV_EINVAL, "%s: packed is NULL or not 16-byte aligned", fn);
  const bool need_anchor = frame0 % cfg->anchor_every != 0;
  if (need_anchor && (!anchor || !aligned16(anchor)))
    return fail(QKV_EINVAL, "%s: frame0 is not an anchor frame: the anchor of its group is required", fn);
  const TLayout L = temporal_layout(cfg, frame0, n_frames);
  TCodecArgs a = tcodec_args(cfg, frame0, n_frames, L);
  a.packed = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(packed));
  a.anchor = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(anchor));
  QKV_HIP(launch_temporal_decode(a, out->ptr, out->dtype == QKV_F32 ? 0 : 1, out->stride_token, out->stride_head,
                                 reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"
