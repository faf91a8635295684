/*
 * libqkv -- KV-cache chunk quantization for autoregressive video models and
 * attention computed directly over the packed cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (cited by page title and section):
 *   [QVG]  "Quant VideoGen: Auto-Regressive Long Video Generation via 2-Bit
 *          KV-Cache Quantization" (paper notes page, ICML 2026).
 *   [QWM]  "AI生成视频时为什么会悄然记错画面？一个被忽视2比特量化陷阱" (summary of
 *          the QuantWM paper).
 *   [TRAP] "视频生成中的2比特量化陷阱：画面为何悄悄失真" (explainer article).
 *   [BLOG] "视频世界模型KV Cache时序稳定2-bit压缩方案实战" (practitioner blog).
 *
 * Conventions for every entry point:
 *   - Return value: a qkv_status.  On failure qkv_last_error() holds a message
 *     (thread-local, valid until the next call on the same thread) and the
 *     outputs are undefined.  Arguments are validated on the host before any
 *     work is enqueued, so a validation failure enqueues nothing.
 *   - Device pointers are plain HIP device addresses, 16-byte aligned.  The
 *     caller owns every buffer (packed chunks, workspaces, outputs); the
 *     library never allocates device memory and keeps no pointer after the
 *     call's work has been enqueued.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is asynchronous; faults surface at the caller's next
 *     synchronisation.  Only qkv_psac_fit synchronises its stream.
 *   - Inputs must be finite; NaN/Inf give unspecified (but memory-safe)
 *     results.
 *   - Calls that share a workspace or a packed chunk on one device must not
 *     overlap in time (they race on it); calls on disjoint buffers may run
 *     concurrently on different streams.
 */
#ifndef QKV_H
#define QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKV_VERSION 1

typedef enum {
  QKV_OK = 0,
  QKV_EINVAL = 1,        /* invalid argument or inconsistent configuration   */
  QKV_EUNSUPPORTED = 2,  /* valid for the method, not built in this library  */
  QKV_EDEVICE = 3,       /* a HIP call failed (message has hipGetErrorString) */
  QKV_EWORKSPACE = 4     /* workspace missing or smaller than required       */
} qkv_status;

typedef enum { QKV_F32 = 0, QKV_BF16 = 1 } qkv_dtype;

/* qkv_config.flags */
#define QKV_FLAG_RTN 1   /* zero centroids, no k-means: plain per-group RTN
                            quantization ([QVG] main table, "RTN" row; the
                            "no clustering" ablation).  For tests/baselines. */

/*
 * Quantizer configuration of one tensor (K or V) of one layer.
 *   head_dim         d; must be 128 (the only head size supported).
 *   n_heads          H in [1, 1024].  Every step is independent per head, so
 *                    layers that share a configuration may be stacked along
 *                    the head axis (H = layers x heads per layer, tensors
 *                    [N][layers * heads][128]): one call then quantizes, and
 *                    one qkv_attend launch attends, all of those layers, with
 *                    each head's results those of its layer alone.
 *   n_clusters       C in [1, 256]: k-means groups per (chunk, head, stage)
 *                    ([QVG] "Semantic-Aware Smoothing").  Needs n_tokens >= C.
 *   kmeans_iters     Lloyd iterations per stage, >= 1 (the fixed protocol
 *                    uses 10): strided init c_j = y[j * floor(N / C)], then
 *                    iters x (assign, update); ties go to the lower index;
 *                    an empty cluster keeps its centroid.
 *   n_stages         L >= 1, <= 4: progressive residual stages ([QVG]
 *                    "Progressive Residual Quantization").
 *   bits             2 or 4: code width of every channel, or of the
 *                    non-sensitive class when n_int4_channels > 0.
 *   group            channels per scale group, a multiple of 16 that divides
 *                    d (uniform layout); in the mixed layout each class is cut
 *                    into runs of `group`, the last run of a class shorter.
 *   n_int4_channels  0 = off.  Otherwise the first n_int4_channels channels of
 *                    the per-head permutation are coded with 4 bits and the
 *                    rest with `bits` (= 2) bits ([TRAP] section five, advice
 *                    one; [BLOG] section 3.2).  Must be in [1, d-1].
 *   psac_rank        r in [0, 8]: PSAC coefficients per key token ([QWM]
 *                    "QuantWM", second technique).  0 = off.
 *   use_qsac         1 = weight k-means distances per channel by w ([QWM]
 *                    "QuantWM", first technique: the channels' query
 *                    activity).  2 = also weigh the dynamic range of the
 *                    residual being quantized (same technique): the weights
 *                    of each stage's k-means are fl32(w_k * fl32(rho_k^2)),
 *                    rho_k = fl32(max - min) of channel k over the chunk's
 *                    tokens of that stage's input (the data, then the
 *                    residual of the previous stages).  0 = off.
 *   flags            QKV_FLAG_*.
 */
typedef struct {
  int32_t head_dim;
  int32_t n_heads;
  int32_t n_clusters;
  int32_t kmeans_iters;
  int32_t n_stages;
  int32_t bits;
  int32_t group;
  int32_t n_int4_channels;
  int32_t psac_rank;
  int32_t use_qsac;
  int32_t flags;
} qkv_config;

/*
 * A strided [n_tokens][n_heads][head_dim] device tensor; the channel
 * dimension is contiguous, strides are in elements, ptr is 16-byte aligned
 * and both strides are multiples of 8.
 */
typedef struct {
  void* ptr;
  int32_t dtype;          /* qkv_dtype */
  int32_t reserved;
  int64_t n_tokens;
  int64_t stride_token;
  int64_t stride_head;
} qkv_tensor;

/*
 * Per-head side inputs of the quantizer (device pointers; NULL when the
 * feature is off):
 *   w     float [H][d]      QSAC channel weights (required when use_qsac > 0).
 *   perm  uint8 [H][d]      channel order, sensitive (4-bit) class first, each
 *                           class listed in the order its channels are packed
 *                           (required when n_int4_channels > 0).
 *   U     float [H][d][r]   PSAC basis, orthonormal columns (required when
 *                           psac_rank > 0).
 */
typedef struct {
  const float* w;
  const uint8_t* perm;
  const float* U;
} qkv_side;

/*
 * Byte layout of one packed chunk of n_tokens tokens (all offsets from the
 * chunk's base pointer, each array 256-byte aligned).  For stage l:
 *   codes     uint32 [H][N][words_per_token] at off_codes + l*stage_bytes_codes.
 *             Stored code u = q + 2^(b-1).  In a class of b-bit channels the
 *             channel at class position p is in word class_word0 + p/(32/b),
 *             bits [b*(p%(32/b)), +b).  The uniform layout has one class in
 *             channel order; the mixed layout has the 4-bit class (words
 *             0..int4_words-1) then the 2-bit class, in perm order.
 *   scales    bf16 [H][N][groups_per_token] at off_scales + l*stage_bytes_scales,
 *             groups in storage order.  S = bf16(fp32(max|r| / (2^(b-1)-1)))
 *             ([QVG] "Research background", core tension).
 *   labels    uint8 [H][N] at off_labels + l*stage_bytes_labels.
 *   centroids bf16 [H][C][d] at off_centroids + l*stage_bytes_centroids
 *             (channel order; [QVG] "Method / Overall framework": centroids
 *             kept in BF16).
 *   perm      uint8 [H][d] at off_perm (mixed layout only, else 0 bytes).
 *   psac      bf16 [H][N][r] at off_psac (psac_rank > 0 only).
 * Dequantization: x_hat = sum over stages of fp32(S*q + C[label]).
 */
typedef struct {
  uint64_t bytes;
  uint64_t off_codes, stage_bytes_codes;
  uint64_t off_scales, stage_bytes_scales;
  uint64_t off_labels, stage_bytes_labels;
  uint64_t off_centroids, stage_bytes_centroids;
  uint64_t off_perm, off_psac;
  int32_t words_per_token;
  int32_t groups_per_token;
  int32_t int4_words;
  int32_t reserved;
  int64_t n_tokens;
} qkv_layout;

int qkv_version(void);
const char* qkv_last_error(void);

/* Host only: validate cfg for chunks of n_tokens tokens and fill *out.
   Errors: QKV_EINVAL / QKV_EUNSUPPORTED for an invalid cfg or n_tokens < C. */
int qkv_chunk_layout(const qkv_config* cfg, int64_t n_tokens, qkv_layout* out);

/* Host only: bytes of device workspace that every entry point below needs for
   chunks of at most max_chunk_tokens tokens, attention over at most n_chunks
   chunks with n_query queries, and qkv_psac_fit with n_query history queries.
   One workspace of this size serves every call with those bounds.  For a
   configuration on the generic decode (several stages, 4-bit codes, or groups
   that are not a multiple of 32) it includes 512 bytes per cached token-head
   for dense fp16 K and V rows, which qkv_attend decodes once per call and
   attends over; given less, qkv_attend decodes inside its tile loop instead
   (the same result up to summation order). */
int qkv_workspace_bytes(const qkv_config* cfg, int64_t max_chunk_tokens, int64_t n_query,
                        int32_t n_chunks, size_t* out);

/*
 * The KV write path for one chunk of one tensor ([QVG] "Method / Overall
 * framework", all stages; [QWM] QSAC and PSAC encode).  x: [N][H][d] bf16 or
 * f32.  Writes the whole packed chunk (layout above) to `packed`, which must
 * hold qkv_chunk_layout(cfg, N).bytes.  side: see qkv_side (may be NULL when
 * no feature needs it).  workspace: qkv_workspace_bytes(cfg, N, 0, 0, ...).
 */
int qkv_quantize_chunk(const qkv_config* cfg, const qkv_tensor* x, const qkv_side* side,
                       void* packed, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The write path of qkv_quantize_chunk ([QVG] "Method / Overall framework")
 * for n independent problems (1 <= n <= 16) in one set of launches, e.g. K
 * and V of a chunk, or several chunks: problem p reads
 * xs[p] and writes packed[p] exactly as qkv_quantize_chunk(cfgs[p], xs[p],
 * sides[p], packed[p], ...) would (sides may be NULL, as may each sides[p]).
 * The problems must share n_heads, n_clusters, kmeans_iters, n_stages and
 * flags of their configs, and n_tokens and dtype of their tensors; bits,
 * group, the mixed layout, QSAC and PSAC may differ.  workspace: at least
 * qkv_quantize_chunks_workspace_bytes(cfgs[0], N, n) bytes, split into one
 * slice per problem.  Errors: QKV_EINVAL for a mismatch or a bad pointer (no
 * work is queued), as qkv_quantize_chunk otherwise.
 */
int qkv_quantize_chunks(int32_t n, const qkv_config* const* cfgs, const qkv_tensor* const* xs,
                        const qkv_side* const* sides, void* const* packed, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Host only: workspace bytes of qkv_quantize_chunks for n problems of
   n_tokens tokens under cfg. */
int qkv_quantize_chunks_workspace_bytes(const qkv_config* cfg, int64_t n_tokens, int32_t n,
                                        size_t* out);

/*
 * qkv_quantize_chunk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The k-means and staging buffers live in a
 * scratch array the library holds on each device (32 MiB, kept until the
 * process ends; looked up on the first call on a device).  Writes the same
 * packed chunk as qkv_quantize_chunk(cfg, x, side, packed, ...).  Calls no
 * allocating routine.  Errors: QKV_EWORKSPACE when the chunk needs more than
 * the scratch array holds (qkv_workspace_bytes(cfg, N, 0, 0) > 32 MiB: e.g.
 * more than one stage at 32 heads x 6,240 tokens), else as qkv_quantize_chunk.
 * All calls on one device share its scratch array: calls that overlap in time
 * on one device (different streams or threads) race on it and must not.
 */
int qkv_quantize_chunk_noalloc(const qkv_config* cfg, const qkv_tensor* x, const qkv_side* side,
                               void* packed, void* stream);

/* Dequantize a packed chunk: out [N][H][d], f32 or bf16 (bf16 = nearest-even
   rounding of the f32 sum).  ([QVG] "Method / Overall framework".) */
int qkv_dequantize(const qkv_config* cfg, int64_t n_tokens, const void* packed,
                   const qkv_tensor* out, void* stream);

/*
 * Attention of queries q [Nq][H][d] (bf16 or f32) over the concatenation of
 * n_chunks packed K chunks and V chunks (device pointers in host arrays
 * k_chunks/v_chunks, token counts in chunk_tokens; chunk i of K and of V hold
 * the same tokens).  ([QVG] "Key designs / algorithm-system co-design":
 * attention reads the packed cache; [QWM] second technique: the PSAC term.)
 *   s_ij = softmax_scale * (q_i . k_hat_j + (q_i U) . coef_j),
 *   out_i = sum_j softmax_j(s_ij) v_hat_j      (out: [Nq][H][d] f32).
 * U: float [H][d][r] device, required iff k_cfg->psac_rank > 0.
 * causal: 1 keeps keys j <= i (token order of the concatenated cache).
 * softmax_scale: 0 selects 1/sqrt(d).
 * logits_debug: NULL, or float [H][Nq][Nk] device receiving s_ij (-inf where
 * masked); for tests.  n_chunks in [1, 1024].
 * Precision and range: decoded keys and values, queries and the PSAC operands
 * enter the matrix cores as fp16 with fp32 accumulation.  A pre-pass reads the
 * largest stored scale, centroid and PSAC coefficient of the call and the
 * largest query, and scales each operand class by a power of two (exact) so
 * that every fp16 operand stays finite; results are scaled back.  There is no
 * bound on the cache's magnitude beyond finite inputs whose logits and outputs
 * fit float32 (operands below the fp16 normal range, 2^-14 after scaling, lose
 * precision gradually).
 */
int qkv_attend(const qkv_config* k_cfg, const qkv_config* v_cfg, const qkv_tensor* q,
               const void* const* k_chunks, const void* const* v_chunks,
               const int64_t* chunk_tokens, int32_t n_chunks, const float* U,
               int32_t causal, float softmax_scale, const qkv_tensor* out,
               float* logits_debug, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One step of autoregressive chunk-by-chunk generation ([QVG] "Research
 * background": causal attention over a resident KV-cache, chunk by chunk; [TRAP]
 * opening: every new frame attends to all cached frames): the queries q
 * [Nf][H][d] (bf16) of a new chunk attend over the n_chunks packed chunks of the
 * cache (as qkv_attend; n_chunks may be 0) followed by the chunk's own keys and
 * values k_fresh, v_fresh [Nf][H][d] (bf16 or f32, unquantized), with a
 * frame-block causal mask: query i sees every cached key and fresh key j iff
 * j / frame_tokens <= i / frame_tokens.  The PSAC term applies to the cached
 * keys only.  Same outputs, softmax_scale, U, logits_debug ([H][Nf][Nk + Nf])
 * and errors as qkv_attend; the workspace of qkv_workspace_bytes(k_cfg,
 * max_chunk_tokens, Nf, n_chunks) covers a fresh chunk of at most
 * max_chunk_tokens tokens.  QKV_EUNSUPPORTED for f32 queries.  The caller then
 * quantizes the chunk (qkv_quantize_chunk(s)) and appends it to the cache.
 */
int qkv_attend_fresh(const qkv_config* k_cfg, const qkv_config* v_cfg, const qkv_tensor* q,
                     const void* const* k_chunks, const void* const* v_chunks, const int64_t* chunk_tokens,
                     int32_t n_chunks, const qkv_tensor* k_fresh, const qkv_tensor* v_fresh,
                     int32_t frame_tokens, const float* U, float softmax_scale, const qkv_tensor* out,
                     float* logits_debug, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Statistics of history queries q_hist [n][n_heads][d] (bf16 or f32) for QSAC and
 * PSAC ([QWM] "QuantWM", both techniques; [TRAP] section five for the
 * ranking):  M_h = sum_n q q^T (float64 on the device);
 *   w_out   float [H][d] device: fp32(M_kk / n) (may be NULL);
 *   U_out   float [H][d][rank] device: eigenvectors of the `rank` largest
 *           eigenvalues of M_h, descending (may be NULL when rank == 0);
 *   perm_out uint8 [H][d] device: the n_int4 largest-w channels ascending,
 *           then the rest ascending (ties -> lower index); NULL or n_int4 == 0
 *           to skip;
 *   energy_out float [H] HOST: top-rank eigenvalue sum / trace (may be NULL).
 * The eigensolver (parallel cyclic Jacobi, float64) runs on the device, one
 * workgroup per head; it stops once the off-diagonal mass is at most 1e-30 of
 * the total, or after 16 sweeps (the room the workspace gives its rotation
 * record).  When rank == 0 and energy_out is NULL only M's diagonal is formed.
 * The host orders the channels from M's diagonal: the call copies it (and the
 * energies) to the host, synchronises `stream`, and returns with w_out and
 * perm_out written.  workspace: qkv_workspace_bytes(cfg, 0, n, 0) bytes.
 */
int qkv_psac_fit(const qkv_tensor* q_hist, int32_t n_heads, int32_t rank, int32_t n_int4,
                 float* U_out, float* w_out, uint8_t* perm_out, float* energy_out,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- Step-level entry points (the steps qkv_quantize_chunk chains) ---- */

/* One k-means assign step ([QVG] "Semantic-Aware Smoothing"):
   labels[h][i] = argmin_j sum_k w_k (y_ik - c_jk)^2 (ties -> lowest j),
   centroids float [H][C][d] device, w float [H][d] or NULL (= all ones),
   labels uint8 [H][N] device. */
int qkv_kmeans_assign(const qkv_config* cfg, const qkv_tensor* y, const float* centroids,
                      const float* w, uint8_t* labels, void* workspace,
                      size_t workspace_bytes, void* stream);

/* One k-means update step: centroids[h][j] = fp32(exact sum / count) of the
   tokens labelled j; an empty cluster keeps its value (in/out).
   counts int32 [H][C] device or NULL.  workspace: qkv_workspace_bytes(cfg, N,
   0, 0, ...) bytes. */
int qkv_kmeans_update(const qkv_config* cfg, const qkv_tensor* y, const uint8_t* labels,
                      float* centroids, int32_t* counts, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Quantize stage `stage` of a packed chunk from given labels and float
   centroids (rounded to bf16 and stored in the chunk): residual, group scale,
   codes ([QVG] core tension formula; "Method / Overall framework").  perm:
   uint8 [H][d] device (mixed layout only; also stored in the chunk).
   y_next: NULL or float [H][N][d] device receiving y - fp32(S*q + C). */
int qkv_quant_pack(const qkv_config* cfg, const qkv_tensor* y, const uint8_t* labels,
                   const float* centroids, const uint8_t* perm, void* packed, int32_t stage,
                   float* y_next, void* stream);

/* ---- Temporally stable 2-bit codec ([BLOG] sections 3.3-3.5) ---- */

/*
 * A second compression scheme, for comparison with the k-means quantizer: per
 * 32-channel block of one token-head, the value of unique largest magnitude
 * (the block's P99 outlier) is kept in fp16 and the others are coded with an
 * fp16 zero point lo = fp16(min) and scale S = fp16((max - lo) / (2^b - 1)),
 * q = clamp(rint((r - lo) / S), 0, 2^b - 1); frame f is an fp16 anchor iff
 * f % anchor_every == 0, every other frame codes r = (kv + feedback) - anchor
 * (its group's anchor as stored, position by position) and rebuilds kv_hat =
 * anchor + (lo + q S); feedback = decay * (kv - kv_hat) carries to the same
 * position of the next frame.  All arithmetic float32, each operation rounded
 * once in that order; fp16 conversions to nearest even.  Inputs within the
 * fp16 range.
 *   n_heads       H in [1, 256] (head_dim 128).
 *   frame_tokens  P >= 1: tokens (positions) per frame.
 *   bits          2 or 4.
 *   anchor_every  >= 1 frames per temporal group ([BLOG] 3.3: 32).
 *   decay         error-feedback decay in [0, 1] ([BLOG] 3.5: 0.8).
 */
typedef struct {
  int32_t n_heads;
  int32_t frame_tokens;
  int32_t bits;
  int32_t anchor_every;
  float decay;
} qkv_tcfg;

/* Bytes of one packed run of n_frames (1 to 64) frames starting at global frame
   frame0 >= 0, and (frame_offsets non-NULL: n_frames entries) each frame's byte
   offset in it.  An anchor frame holds fp16 values [P][H][128]; any other frame
   holds, each section 256-byte aligned in this order: codes u32 [P][H][4 * bits]
   (channel k of block j of a token-head in word j * bits + k / (32 / bits),
   bits * (k % (32 / bits)) up), lo fp16 [P][H][4], scale fp16 [P][H][4],
   outlier value fp16 [P][H][4] (0 when none), outlier channel within the block
   u8 [P][H][4] (255 when none).  Host only. */
int qkv_temporal_layout(const qkv_tcfg* cfg, int64_t frame0, int32_t n_frames, size_t* bytes,
                        size_t* frame_offsets);

/* Bytes of the state carried from one call to the next: feedback f32
   [P][H][128], then (at offset 4 * P * H * 128) the current anchor fp16
   [P][H][128].  Host only. */
int qkv_temporal_state_bytes(const qkv_tcfg* cfg, size_t* bytes);

/* Code frames frame0 .. frame0 + n_frames - 1 of x [n_frames * P][H][128] (bf16
   or f32; frame by frame, each frame's P tokens in position order) into packed
   (qkv_temporal_layout bytes, device), serially over frames.  state (device,
   qkv_temporal_state_bytes): read unless frame0 is an anchor frame (the start
   of a stream must be one), then replaced by the state after the last frame. */
int qkv_temporal_encode(const qkv_tcfg* cfg, const qkv_tensor* x, int64_t frame0, void* state, void* packed,
                        void* stream);

/* Rebuild out [n_frames * P][H][128] (f32 or bf16, rounded to nearest even)
   from a run packed by qkv_temporal_encode (same frame0 and n_frames).
   anchor: fp16 [P][H][128] device, the anchor of frame0's group as stored (the
   anchor section of the state before the run was coded, or that anchor frame's
   packed values); unused, and may be NULL, when frame0 is an anchor frame. */
int qkv_temporal_decode(const qkv_tcfg* cfg, int64_t frame0, int32_t n_frames, const void* packed,
                        const void* anchor, const qkv_tensor* out, void* stream);

/* ---- Kernel timing, for measurement tools ---- */

/* Per-kernel totals returned by qkv_timing_read. */
typedef struct {
  char name[32];        /* kernel name, e.g. "k_assign", NUL-terminated */
  int64_t launches;
  double total_ms;      /* sum of the event-measured durations */
} qkv_kernel_time;

/* on = 1: from now on every kernel launch of the library (on any thread) is
   bracketed by HIP events on its stream, and the record starts empty; on = 0:
   stop recording.  The events add a few microseconds between launches; timed
   runs that report throughput leave this off.  Host only; always QKV_OK. */
int qkv_timing_enable(int32_t on);

/* Waits for every recorded launch and writes per-kernel totals (sorted by
   name) to out[0 .. min(n, max_kernels)), n = the number of distinct kernels
   (*n_out).  Errors: QKV_EINVAL for a NULL n_out (or out with max_kernels >
   0), QKV_EDEVICE when an event cannot be read. */
int qkv_timing_read(int32_t max_kernels, qkv_kernel_time* out, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* QKV_H */
