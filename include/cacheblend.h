/*
 * cacheblend.h -- C ABI of the CacheBlend per-layer KV fusor for MI355X (gfx950).
 *
 * The fusor is the GPU part of CacheBlend ("CacheBlend: Fast Large Language
 * Model Serving for RAG with Cached Knowledge Fusion", arXiv 2405.16444).
 * Every retrieved chunk has a KV cache computed on its own at positions
 * 0 .. L_c-1.  At query time the chunks are laid out in context order, the
 * cached keys are moved to their new absolute positions, and on every layer
 * a small set of tokens is recomputed (section 4.2, Figure 5b): the layer
 * input is masked down to the selected tokens, their Q/K/V are computed, the
 * K/V of the other tokens are reused from the cache, and attention of the
 * selected tokens over all tokens produces the next layer's input.  The
 * tokens are the ones with the highest KV deviation (HKVD, section 4.3),
 * narrowed gradually from layer to layer (section 4.3, Figure 9).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Geometry.  The context is n_chunks chunks in context order followed by
 *    the query.  Row (token) j of the context has global position j.  Chunk c
 *    occupies rows [o_c, o_{c+1}) with o_0 = 0 and o_{n_chunks} = n_ctx; the
 *    query rows are [n_ctx, T).  The first chunk is the prefix: its cached KV
 *    is exact and it is never re-rotated nor recomputed.  The candidate rows
 *    for recomputation are [first_chunk_len, n_ctx).
 *  - Tensors are row-major.  Caches are [T][n_kv_heads][head_dim]; hidden
 *    states are [rows][d_model]; weights are in nn.Linear layout
 *    [out_features][in_features]: w_q [n_q*hd][d], w_k/w_v [n_kv*hd][d],
 *    w_o [d][n_q*hd], w_gate/w_up [ffn][d], w_down [d][ffn].  Element type is
 *    cb_layer_config.dtype (bf16 or fp32) for weights, caches and hidden
 *    states; RMSNorm gains and RoPE tables are always fp32.
 *  - RoPE (section 4.3, footnote 3, and the aifetchly guide, "RoPE Delta
 *    Positional Realignment"): interleaved pairs (2i, 2i+1) of every head are
 *    rotated by angle p*theta_i, theta_i = rope_theta^(-2i/hd).  Kernels read
 *    cos/sin from a device table cb_rope_dev built by cb_rope_table on the
 *    host (fp64 angle, C library cos/sin, rounded once to fp32).
 *  - Pointers marked "device" are HIP device pointers; "host" pointers are
 *    read before the call returns.  The library allocates no memory: every
 *    buffer, including the workspace, belongs to the caller and no pointer is
 *    kept after the call, except by work still in flight on `stream`.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every device call only enqueues work on it and returns without a device
 *    synchronisation; results are ready when the stream has drained.
 *  - Errors are returned as cb_status; nothing aborts or throws across the
 *    ABI.  Argument and shape checks happen on the host before anything is
 *    enqueued.  Device index arrays are not read on the host (unless validate
 *    mode is on, cb_set_validate): out-of-range entries are skipped by the
 *    kernels' bounds checks and make the results unspecified, never an
 *    out-of-bounds access.  A failed HIP launch returns CB_ERR_HIP and its
 *    code is kept per thread (cb_last_hip_error).
 *  - Calls that share a workspace or a cache must not overlap in time.
 */
#ifndef CACHEBLEND_H
#define CACHEBLEND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CB_OK = 0,
  CB_ERR_ARG = 1,          /* null pointer, negative size, bad enum            */
  CB_ERR_SHAPE = 2,        /* inconsistent geometry or head layout             */
  CB_ERR_INDEX = 3,        /* an index array failed validation (validate mode) */
  CB_ERR_WORKSPACE = 4,    /* workspace smaller than cb_workspace_size()       */
  CB_ERR_UNSUPPORTED = 5,  /* shape the gfx950 kernels do not handle           */
  CB_ERR_HIP = 6           /* a HIP runtime call or launch failed              */
} cb_status;

typedef enum { CB_F32 = 0, CB_BF16 = 1 } cb_dtype;

/* Shape of one Llama-style decoder layer (no biases, RMSNorm, GQA, SwiGLU).
 * Requirements: n_q_heads % n_kv_heads == 0; head_dim a multiple of 8.  bf16 needs
 * head_dim in {64, 128}, n_q_heads / n_kv_heads in {1, 2, 4, 8} and d_model,
 * ffn_dim multiples of 8.  fp32 needs head_dim <= 256. */
typedef struct {
  int32_t d_model;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn_dim;
  float rope_theta;
  float rms_eps;
  int32_t dtype;           /* cb_dtype */
} cb_layer_config;

/* Device pointers to one layer's weights (layouts above).  attn_norm and
 * mlp_norm are fp32 [d_model].  w_gateup_packed is optional (NULL = unused):
 * W_gate and W_up repacked once by cb_pack_gateup, which the bf16 gate/up
 * projection then streams instead of w_gate and w_up (same results, bit for
 * bit).  w_qkv_folded is optional (NULL = unused): [W_q; W_k; W_v] with the
 * attention RMSNorm gain folded in (cb_fold_qkv); with it the bf16 calls run
 * the attention RMSNorm inside the QKV projection (the raw input rows are
 * projected and each row's product is scaled by its 1 / rms, section 4.2's
 * mask-then-project in one pass) instead of as a separate pass.  Results
 * then differ from the unfolded path by rounding only (the normalised rows
 * are not rounded to bf16 before the product; the folded weights are). */
typedef struct {
  const void* attn_norm;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_o;
  const void* mlp_norm;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* w_gateup_packed;
  const void* w_qkv_folded;
} cb_layer_weights;

/* Device RoPE table: cos[p][hd/2], sin[p][hd/2] fp32 for p = 0 .. n_pos-1,
 * as written by cb_rope_table(cfg, 0, n_pos, ...) and copied to the device.
 * head_dim and rope_theta name the configuration the table was built for;
 * every call that takes a table returns CB_ERR_ARG unless both equal the
 * call's cfg (a table of another base or head size would rotate by the
 * wrong angles) and cos and sin are 16-byte aligned, and CB_ERR_SHAPE when
 * n_pos is below the positions the call reads. */
typedef struct {
  const float* cos;
  const float* sin;
  int32_t n_pos;
  int32_t head_dim;
  float rope_theta;
} cb_rope_dev;

/* ---------------------------------------------------------------------------
 * Host helpers
 * ------------------------------------------------------------------------- */

/* RoPE table for positions pos_begin .. pos_begin+n_pos-1 into HOST buffers
 * cos_out/sin_out [n_pos][head_dim/2] (CacheBlend section 4.3, footnote 3:
 * the rotation matrix of angle m*theta).  theta_i = pow(rope_theta, -2i/hd)
 * and angle = p * theta_i are evaluated in fp64 and cos/sin are rounded once
 * to fp32 (round to nearest even).  CB_ERR_ARG on null or negative input. */
cb_status cb_rope_table(const cb_layer_config* cfg, int32_t pos_begin, int32_t n_pos,
                        float* cos_out, float* sin_out);

/* Number of HKVD tokens for a recompute ratio r = r_e4 / 10000 over n_ctx
 * context tokens (section 4.2: recomputing r% of the tokens): min(ceil(r *
 * n_ctx), n_cand), in exact integer arithmetic.  -1 on negative input. */
int32_t cb_num_selected(int32_t r_e4, int32_t n_ctx, int32_t n_cand);

/* Gradual filtering schedule (section 4.3, Figure 9) into HOST k_out[n_layers]:
 * layer 0 recomputes every candidate (k_out[0] = n_cand); layer l >= 1 keeps
 * ceil(r_l * n_ctx) tokens with r_l falling linearly from r_first (l = 1) to
 * r_last (l = n_layers-1); r_last_e4 == 0 keeps r_first on every layer.  k
 * never grows from one layer to the next. */
cb_status cb_filter_schedule(int32_t n_layers, int32_t r_first_e4, int32_t r_last_e4,
                             int32_t n_ctx, int32_t n_cand, int32_t* k_out);

/* One-time weight repack (a model-load step, not part of a request).  The
 * gate/up projection streams 224-row tiles (112 gate rows, then the same 112
 * up rows) in 32-element K steps; cb_pack_gateup stores W_gate and W_up (bf16
 * device [ffn][d] each) in exactly that order, tile by tile and step by step,
 * each (tile, step) block of 224 rows x 64 bytes contiguous, rows past ffn
 * and K past d zero, so that every load of the kernel reads contiguous
 * memory (d_model a multiple of 128; otherwise the projection reads the
 * row-major weights).  packed: device, cb_pack_gateup_size(cfg) bytes, 16-byte aligned.
 * CB_ERR_UNSUPPORTED for fp32 configs (the fp32 path does not use it). */
size_t cb_pack_gateup_size(const cb_layer_config* cfg);
cb_status cb_pack_gateup(const cb_layer_config* cfg, const void* w_gate, const void* w_up,
                         void* packed, void* stream);

/* One-time fold of the attention RMSNorm gain into the QKV weights (a
 * model-load step): out[r][k] = W[r][k] * attn_norm[k] rounded to bf16 for
 * the rows r of W_q, then W_k, then W_v (device, cb_fold_qkv_size(cfg)
 * bytes, 16-byte aligned).  Reads w->w_q, w_k, w_v and attn_norm.
 * CB_ERR_UNSUPPORTED for fp32 configs (cb_fold_qkv_size is then 0). */
size_t cb_fold_qkv_size(const cb_layer_config* cfg);
cb_status cb_fold_qkv(const cb_layer_config* cfg, const cb_layer_weights* w, void* out, void* stream);

/* Bytes of device workspace needed by cb_blend_layer with up to m_max input
 * rows and by cb_full_prefill_layer with T <= m_max rows, and by
 * cb_select_hkvd with n <= m_max candidates.  0 on invalid cfg. */
size_t cb_workspace_size(const cb_layer_config* cfg, int32_t T, int32_t m_max);

/* Bytes of device workspace needed by cb_blend_stack over T rows: the
 * per-layer workspace of cb_workspace_size(cfg, T, T), two [T][d] hidden
 * buffers, a [T] row list and two staging slots for one layer's 8-bit K/V
 * (cb_blend_stack_kv8).  0 on invalid cfg or T <= 0. */
size_t cb_stack_workspace_size(const cb_layer_config* cfg, int32_t T);

/* Loading controller of section 5: the recompute ratio of one layer, in
 * units of 1e-4.  The recompute delay of ratio r is modelled as r x
 * t_prefill_us, the offline-profiled full prefill of one layer over the
 * context (footnote 5); the load delay of one layer's KV as
 * kv_bytes_per_token x n_tokens / link_bytes_per_us (footnote 6).  The ratio
 * at which the two delays are equal, r_match = load / prefill, is rounded
 * down to a multiple of 1e-4 (so the recompute stays within the load time)
 * and capped at 1; the result is max(that, r_min_e4), the smallest ratio
 * whose quality loss is negligible (the paper finds 15%, Figure 16).
 * Returns -1 if a time, size or rate is not positive and finite, n_tokens
 * <= 0, or r_min_e4 is outside [0, 10000]. */
int32_t cb_pick_ratio(double t_prefill_us, double kv_bytes_per_token, int32_t n_tokens,
                      double link_bytes_per_us, int32_t r_min_e4);

const char* cb_status_string(cb_status s);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int32_t cb_last_hip_error(void);

/* Validate mode for the calls this thread makes (off by default); returns
 * the previous setting.  When on, cb_blend_layer, cb_blend_layer_fp8,
 * cb_blend_batch and cb_select_hkvd first copy their device index arrays
 * to the host (synchronising `stream`, since earlier work on it may produce
 * them) and check them before enqueuing anything: CB_ERR_INDEX when s_in is
 * not strictly ascending, has a row below first_chunk_len or at/after T, or
 * lacks one of the query rows n_ctx .. T-1, when an in_rows entry is outside
 * [0, T), or when a cand_rows entry is outside [0, T); CB_ERR_ARG when a
 * deviation array given as input (k_new == NULL) holds a NaN (section 4.3's
 * ranking needs ordered values). */
int32_t cb_set_validate(int32_t on);

/* Kernel timing.  Between cb_profile_begin and cb_profile_end every kernel
 * the library launches from this thread is bracketed by two hipEvents
 * recorded on its stream (events are created on first use and reused; no
 * device memory is allocated).  cb_profile_end waits for those events and
 * writes one record per kernel name (up to max_out) to out (host); it returns
 * the number of distinct names, or -1 if an event could not be read. */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
  double min_ms;
  double max_ms;
} cb_kernel_stat;

cb_status cb_profile_begin(void);
int32_t cb_profile_end(cb_kernel_stat* out, int32_t max_out);

/* ---------------------------------------------------------------------------
 * Deviation analytics (diagnostics around the fusor, not steps of it;
 * section 4.1 attention deviation, Figure 7 deviation concentration,
 * section 4.3 / Figure 8 rank correlation across layers)
 * ------------------------------------------------------------------------- */

/* Byte offset in a workspace where cb_blend_layer (called with this T) and
 * cb_full_prefill_layer (over T rows) leave the Q of the rows they
 * recomputed: [rows][n_q_heads * head_dim] in cfg->dtype, RoPE applied at
 * each row's position, rows in the order of s_in (blend; the query rows are
 * the last T - n_ctx) or 0 .. T-1 (full prefill).  Valid until the next call
 * that uses the workspace.  0 on invalid cfg or T <= 0. */
size_t cb_workspace_q_offset(const cb_layer_config* cfg, int32_t T);

/* Workspace bytes for cb_attention_deviation over m rows of n_q heads and for
 * cb_spearman / cb_top_share over n values (the larger of the two). */
size_t cb_analytics_workspace_size(int32_t m, int32_t n_q, int32_t n);

/* Attention deviation (section 4.1): with A_x[i][h][t] = softmax over
 * t <= last_key[i] of q_x[i,h] . k_x[t, h / (n_q/n_kv)] / sqrt(head_dim) and
 * 0 for t > last_key[i], writes out[0] = ||A_a - A_b||_F^2 and out[1] =
 * ||A_b||_F^2 (device double [2]; the relative deviation is
 * sqrt(out[0] / out[1])).  q_a, q_b: device [m][n_q][hd]; k_a, k_b: device
 * [T][n_kv][hd] (cfg dtype); last_key: device int32 [m], clamped to
 * [0, T-1].  Scores and probabilities in fp32, sums in fp64 in a fixed
 * order.  ws: device, >= cb_analytics_workspace_size(m, n_q, 0) bytes. */
cb_status cb_attention_deviation(const cb_layer_config* cfg, int32_t m, const void* q_a, const void* k_a,
                                 const void* q_b, const void* k_b, int32_t T, const int32_t* last_key,
                                 double* out, void* ws, size_t ws_bytes, void* stream);

/* Spearman's rank correlation of x and y (device fp32 [n], finite values):
 * Pearson's correlation of their average ranks (tied values share the mean
 * of the ranks they span), fp64, written to out (device double [1]; NaN
 * when a rank vector is constant).  ws >= cb_analytics_workspace_size(0, 0,
 * n) bytes. */
cb_status cb_spearman(const float* x, const float* y, int32_t n, double* out, void* ws, size_t ws_bytes,
                      void* stream);

/* Share of sum(x) held by the k largest values of x (device fp32 [n],
 * finite; 0 <= k <= n): out[0] (device double) = that sum / sum(x), NaN when
 * sum(x) <= 0.  ws >= cb_analytics_workspace_size(0, 0, n) bytes. */
cb_status cb_top_share(const float* x, int32_t n, int32_t k, double* out, void* ws, size_t ws_bytes,
                       void* stream);

/* Measurement reference (not a step of the fusor): copies `bytes` bytes from
 * src to dst (device, 16-byte aligned, bytes a multiple of 16; CB_ERR_ARG
 * otherwise; the ranges must not overlap) with a plain streaming kernel:
 * 16-byte accesses, each wave instruction over 1 KB of contiguous memory,
 * non-temporal stores.  Its rate on large, cold buffers is the HBM ceiling
 * the bandwidth-bound calls (cb_rope_shift, the deviation of cb_select_hkvd,
 * cb_kv_from_fp8) are compared with.  Asynchronous on `stream`. */
cb_status cb_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Device calls
 * ------------------------------------------------------------------------- */

/* RoPE position re-alignment of cached keys (section 4.3, footnote 3; the
 * aifetchly guide: R(m + delta) = R(delta) R(m), values untouched).
 * k_cache: device, n_layers buffers [T][n_kv][hd], buffer l at element offset
 * l * layer_stride_elems; modified in place.  chunk_offsets: host int32
 * [n_chunks+1], non-decreasing, chunk_offsets[0] = 0, chunk_offsets[n_chunks]
 * = n_ctx <= T.  Every row of chunk c >= 1 is rotated once more by delta =
 * chunk_offsets[c]; rows of chunk 0 and query rows are not touched.  The
 * rotation is done in fp32 as two rounded products and one rounded sum per
 * output, then stored in the cache dtype (round to nearest even).
 * Needs rope->n_pos > chunk_offsets[n_chunks-1]; 1 <= n_chunks <= 256. */
cb_status cb_rope_shift(const cb_layer_config* cfg, const cb_rope_dev* rope, void* k_cache,
                        int64_t layer_stride_elems, int32_t n_layers, int32_t T,
                        const int32_t* chunk_offsets, int32_t n_chunks, void* stream);

/* HKVD selection (section 4.1 KV deviation, section 4.3 top tokens).
 * n candidates, candidate i has token id cand_rows[i] (device int32 [n],
 * strictly ascending; NULL means token id i).
 * If k_new != NULL (device [n][n_kv][hd], cfg dtype): dev[i] = squared L2 norm
 * over all KV heads of k_new[i] - k_ref[cand_rows[i]] (k_ref device [T][n_kv]
 * [hd]), computed in fp32 from the stored values, is written to dev (device
 * fp32 [n]).  If k_new == NULL, dev is an input.  The k largest deviations,
 * ranked by (deviation descending, candidate index ascending), are written
 * to sel_out (device int32 [k]) as token ids in ascending order.
 * 0 <= k <= n; workspace >= cb_workspace_size(cfg, T, n). */
cb_status cb_select_hkvd(const cb_layer_config* cfg, const void* k_new, const void* k_ref,
                         int32_t T, const int32_t* cand_rows, int32_t n, int32_t k, float* dev,
                         int32_t* sel_out, void* ws, size_t ws_bytes, void* stream);

/* One layer of selective KV recompute (section 4.2, Figure 5b; HKVD
 * selection of section 4.3).
 *  k_cache, v_cache: device [T][n_kv][hd], this layer's cache with keys
 *      already at their absolute positions (cb_rope_shift).  The new K/V of
 *      every row of s_in are written in place; other rows are not touched.
 *  s_in: device int32 [m_in], strictly ascending token ids, all >= first_
 *      chunk_len; its last T - n_ctx entries are the query rows n_ctx..T-1.
 *  hidden_in: device [*][d]; row in_rows[i] (device int32 [m_in]; NULL means
 *      row i) is the layer input of token s_in[i].
 *  k_out: how many candidates (s_in entries < n_ctx) to keep.  The kept set
 *      s_out is the k_out candidates of largest K deviation (squared L2 of new
 *      minus cached K over all KV heads, read before the cache row is
 *      replaced), ranked by (deviation desc, token id asc), plus every query
 *      row, in ascending token order.  If k_out >= the candidate count, s_out
 *      = s_in.  m_out = min(k_out, m_in - (T - n_ctx)) + (T - n_ctx) is
 *      written to *m_out_host (host, may be NULL) before the call returns.
 *  Outputs (device): hidden_out [m_out][d] (the layer output of the kept
 *      rows, in s_out order), dev_out fp32 [m_in] (NaN on query rows; may be
 *      NULL), s_out int32 [m_out].  Attention of each kept row j is causal
 *      over cache rows 0..j of the blended cache.
 *  hidden_in must not alias hidden_out.
 *  Workspace >= cb_workspace_size(cfg, T, m_in). */
cb_status cb_blend_layer(const cb_layer_config* cfg, const cb_layer_weights* w,
                         const cb_rope_dev* rope, void* k_cache, void* v_cache, int32_t T,
                         int32_t n_ctx, int32_t first_chunk_len, const int32_t* s_in,
                         int32_t m_in, const void* hidden_in, const int32_t* in_rows,
                         int32_t k_out, void* hidden_out, float* dev_out, int32_t* s_out,
                         int32_t* m_out_host, void* ws, size_t ws_bytes, void* stream);

/* One layer of the fusor from a cache whose keys are still at their chunk-
 * local positions: the re-alignment of cb_rope_shift (section 4.3, footnote
 * 3) and the selective recompute of cb_blend_layer (section 4.2, Figure 5b)
 * in one call.  The results -- cache, hidden_out, dev_out, s_out, m_out --
 * are bit for bit those of cb_rope_shift(cfg, rope, k_cache, 0, 1, T,
 * chunk_offsets, n_chunks, stream) followed by cb_blend_layer with n_ctx =
 * chunk_offsets[n_chunks] and first_chunk_len = chunk_offsets[1] (n_ctx when
 * n_chunks = 1).  Rows of chunks >= 1 that are not in s_in are re-aligned;
 * rows in s_in get their new K/V (their deviation is taken against the
 * re-aligned cached key).  On the bf16 path without split-K the
 * re-alignment runs in the QKV projection's launch, on CUs the projection
 * leaves idle; otherwise it is a launch of its own before the projection.
 *  chunk_offsets: host int32 [n_chunks+1] as for cb_rope_shift (1 <=
 *      n_chunks <= 256, CB_ERR_ARG for NULL or n_chunks < 1,
 *      CB_ERR_UNSUPPORTED above 256, CB_ERR_SHAPE if not non-decreasing from
 *      0 or chunk_offsets[n_chunks] > T).
 *  Every other argument, its checks and the workspace are those of
 *  cb_blend_layer.  The caller keeps ownership of every buffer. */
cb_status cb_blend_layer_realign(const cb_layer_config* cfg, const cb_layer_weights* w,
                                 const cb_rope_dev* rope, void* k_cache, void* v_cache, int32_t T,
                                 const int32_t* chunk_offsets, int32_t n_chunks,
                                 const int32_t* s_in, int32_t m_in, const void* hidden_in,
                                 const int32_t* in_rows, int32_t k_out, void* hidden_out,
                                 float* dev_out, int32_t* s_out, int32_t* m_out_host, void* ws,
                                 size_t ws_bytes, void* stream);

/* The ordinary decoder layer over T rows at positions pos0 .. pos0+T-1 (the
 * "full KV recompute" baseline of section 7 and the isolated precompute of a
 * chunk at position 0).  hidden_in device [T][d]; k_out, v_out device
 * [T][n_kv][hd] receive the layer's K (rotated) and V; hidden_out device
 * [T][d].  Attention of row i is causal over rows 0..i.
 * Workspace >= cb_workspace_size(cfg, T, T). */
cb_status cb_full_prefill_layer(const cb_layer_config* cfg, const cb_layer_weights* w,
                                const cb_rope_dev* rope, const void* hidden_in, int32_t T,
                                int32_t pos0, void* k_out, void* v_out, void* hidden_out,
                                void* ws, size_t ws_bytes, void* stream);

/* One request of a batched fusor layer (cb_blend_batch): its own cache and
 * geometry, as the arguments of the same name of cb_blend_layer. */
typedef struct {
  void* k_cache;             /* device [T][n_kv][hd], updated in place */
  void* v_cache;
  int32_t T;
  int32_t n_ctx;
  int32_t first_chunk_len;
  int32_t m_in;              /* rows this request recomputes */
  int32_t k_out;
} cb_blend_request;

/* One fusor layer for several requests at once: their recomputed rows are
 * stacked into one set of projections (raising the row count of every GEMM),
 * while the K deviation, the scatter, the top-k and the attention of each
 * row use its own request's cache and geometry (section 4.2, Figure 5b, per
 * request; section 7 measures throughput under many concurrent requests,
 * Figure 14, and prefill time against batch size, Figure 15c).  For every request the result equals cb_blend_layer
 * on that request alone, up to the rounding order of the attention key split
 * (the split is chosen from the batch's row count).
 *  reqs: host [n_req], 1 <= n_req <= 16.  m_out_r = min(k_out_r, m_in_r - q_r)
 *    + q_r with q_r = T_r - n_ctx_r (host-computable).
 *  s_in: device int32 [sum m_in]; request r's rows (ascending positions in
 *    its own cache, every query row, none below first_chunk_len) at offset
 *    sum_{j<r} m_in_j.  hidden_in: device [sum m_in][d], row i the input of
 *    s_in[i].  hidden_out: device [sum m_out][d] and s_out: device int32
 *    [sum m_out], request r's kept rows at offset sum_{j<r} m_out_j.
 *    dev_out: device fp32 [sum m_in] or NULL.  m_out_host: host [n_req] or
 *    NULL.
 *  Workspace >= cb_workspace_size(cfg, max_r T_r, sum_r m_in_r); rope covers
 *  max_r T_r positions.  CB_ERR_UNSUPPORTED for n_req > 16; other errors as
 *  cb_blend_layer. */
cb_status cb_blend_batch(const cb_layer_config* cfg, const cb_layer_weights* w,
                         const cb_rope_dev* rope, int32_t n_req, const cb_blend_request* reqs,
                         const int32_t* s_in, const void* hidden_in, void* hidden_out,
                         float* dev_out, int32_t* s_out, int32_t* m_out_host, void* ws,
                         size_t ws_bytes, void* stream);

/* 8-bit float operands (the paper serves its larger models with 8-bit
 * weights, section 7): OCP fp8 E4M3 codes (bias 7, largest finite 448, no
 * infinities) with one power-of-two scale per row.
 *
 * cb_quantize_fp8: x device [rows][cols] (src_dtype CB_F32 or CB_BF16) ->
 * codes device uint8 [rows][cols] and exps device int32 [rows], where
 * exps[i] is the smallest integer e with max_j |x[i][j]| <= 448 * 2^e (0 for
 * an all-zero row) and codes[i][j] is x[i][j] * 2^-e (exact) clamped to +-448
 * and rounded to the nearest E4M3 value, ties to even. */
cb_status cb_quantize_fp8(int32_t src_dtype, const void* x, int32_t rows, int32_t cols,
                          uint8_t* codes, int32_t* exps, void* stream);

/* Bytes of workspace cb_gemm_fp8 needs for these sizes (0 = none). */
size_t cb_gemm_fp8_workspace_size(int32_t M, int32_t N, int32_t K);

/* C[i][j] = sum_k A[i][k] B[j][k] * 2^(a_exp[i] + b_exp[j]) for E4M3 codes A
 * device [M][K] and B device [N][K] (nn.Linear layout), row exponents as
 * produced by cb_quantize_fp8; products are exact and accumulate in fp32.
 * c device [M][ldc] (out_dtype CB_F32 or CB_BF16, rounded once).  K must be a
 * multiple of 16 and A, B 16-byte aligned (CB_ERR_SHAPE); M*K and N*K below
 * 2^31 (CB_ERR_UNSUPPORTED).  ws: device, >= cb_gemm_fp8_workspace_size
 * bytes (may be NULL when that is 0). */
cb_status cb_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* a, const int32_t* a_exp,
                      const uint8_t* b, const int32_t* b_exp, void* c, int32_t ldc, int32_t out_dtype,
                      void* ws, size_t ws_bytes, void* stream);

/* cb_gemm_fp8 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same product, the same kernels and the same bits as cb_gemm_fp8; the
 * split-K partials that cb_gemm_fp8 keeps in the caller's workspace live
 * instead in a static device array of CB_GEMM_FP8_SCRATCH_BYTES inside the
 * library, one copy per GPU, held until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); the
 * device address of the current device's copy is looked up once per device,
 * on the first call made with that device current.
 *  Arguments, layouts and results as cb_gemm_fp8; `stream` must belong to
 *  the current device.  CB_ERR_WORKSPACE when the partials
 *  (cb_gemm_fp8_workspace_size(M, N, K) bytes) exceed the static array;
 *  other errors as cb_gemm_fp8.  Every call on one GPU shares that GPU's
 *  array: calls whose work overlaps in time on one GPU (different streams,
 *  or different host threads, without ordering between them) race on it and
 *  give unspecified results.  Calls ordered on one stream are safe. */
#define CB_GEMM_FP8_SCRATCH_BYTES (32u << 20)
cb_status cb_gemm_fp8_noalloc(int32_t M, int32_t N, int32_t K, const uint8_t* a, const int32_t* a_exp,
                              const uint8_t* b, const int32_t* b_exp, void* c, int32_t ldc,
                              int32_t out_dtype, void* stream);

/* The fusor over a stack of n_layers layers (section 4.3, Figure 9), with
 * each layer's KV loaded while the previous layer is recomputed (section 5,
 * Figure 11: the fusor waits for the previous layer's recompute and for the
 * layer's KV in GPU memory, then recomputes).
 *  layers: host [n_layers] weight sets.  ks: host [n_layers] k_out per layer
 *    (cb_filter_schedule).  Layer 0 recomputes every row from
 *    first_chunk_len = chunk_offsets[1] (n_ctx when n_chunks = 1) to T-1;
 *    layer l > 0 recomputes the rows layer l-1 kept.  Row counts: m_in_0 =
 *    T - first_chunk_len; m_out_l = min(ks[l], m_in_l - q) + q with q =
 *    T - n_ctx; m_in_{l+1} = m_out_l.  If m_rows_host is not NULL it
 *    receives m_in_l, m_out_l for every layer (host [2*n_layers]).
 *  k_caches, v_caches: device; layer l's cache [T][n_kv][hd] at element
 *    offset l * layer_stride_elems.  On return (once the streams drain)
 *    they hold the blended K/V of every layer.
 *  k_src, v_src: both NULL, or both host [n_layers][T][n_kv][hd] (layer
 *    stride T*n_kv*hd, allocate with hipHostMalloc for asynchronous copies)
 *    holding each layer's chunk KV in context order.  When given, layer l's
 *    K and V are copied into the device caches on copy_stream and layer l's
 *    work on `stream` waits for those copies only; the copies of later
 *    layers overlap the recompute.  copy_stream NULL = the copies run on
 *    `stream`, in order, with no overlap.  The copies wait for work already
 *    queued on `stream`.  When NULL, the device caches already hold the
 *    chunk KV.
 *  shift: nonzero = the chunk keys are at their local positions and are
 *    re-aligned first (as cb_rope_shift; per layer after its copy when
 *    loading, one launch over all layers otherwise); 0 = already aligned.
 *  x_first: device [T - first_chunk_len][d], layer 0's input rows.
 *  s_out_all: device int32 [sum_l m_out_l], layer l's kept rows at offset
 *    sum_{j<l} m_out_j (ascending; layer l+1's input rows).
 *  dev_all: device fp32 [sum_l m_in_l], layer l's deviations at offset
 *    sum_{j<l} m_in_j (as dev_out of cb_blend_layer).
 *  hidden_out: device [m_out_{n_layers-1}][d], the last layer's output for
 *    its kept rows.
 *  Workspace >= cb_stack_workspace_size(cfg, T).  The call creates and
 *  releases one HIP event per layer (host objects; no device memory).
 *  Errors as cb_blend_layer; nothing is enqueued when a check fails. */
cb_status cb_blend_stack(const cb_layer_config* cfg, int32_t n_layers, const cb_layer_weights* layers,
                         const cb_rope_dev* rope, void* k_caches, void* v_caches,
                         int64_t layer_stride_elems, const void* k_src, const void* v_src, int32_t T,
                         const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift,
                         const void* x_first, const int32_t* ks, int32_t* s_out_all, float* dev_all,
                         void* hidden_out, int32_t* m_rows_host, void* ws, size_t ws_bytes,
                         void* stream, void* copy_stream);

/* 8-bit stored chunk KV.  The paper serves its larger models with 8-bit
 * weights (section 7); the same E4M3 format halves the bytes of the stored
 * KV that the loader of section 5 moves (one power-of-two exponent per
 * (token, KV head) row of head_dim values, as cb_quantize_fp8 produces over
 * rows of head_dim).
 *
 * cb_kv_from_fp8: expands codes into the caches, K and V of rows
 * row_begin .. row_begin+n_rows-1 of n_layers layers:
 *  k_codes, v_codes: device uint8 [n_layers][n_rows][n_kv][hd], 16-byte
 *    aligned; k_exps, v_exps: device int32 [n_layers][n_rows][n_kv].
 *  k_cache, v_cache: device [T][n_kv][hd] in cfg->dtype, layer l at element
 *    offset l * layer_stride_elems.  Written: value(code) * 2^exp, exact in
 *    fp32 and bf16; with shift != 0 the keys of rows in chunk c >= 1 are
 *    then rotated by delta = chunk_offsets[c] exactly as cb_rope_shift does
 *    (the same bits as expanding and then shifting).  Other rows untouched.
 *  chunk_offsets: host [n_chunks+1] as cb_rope_shift (n_chunks <= 256).
 *  rope: device tables covering chunk_offsets[n_chunks-1] + 1 positions
 *    (only read, and only checked, when shift != 0).
 *  CB_ERR_SHAPE when hd is not a multiple of 16 or rows exceed T; other
 *  errors as cb_rope_shift. */
cb_status cb_kv_from_fp8(const cb_layer_config* cfg, const cb_rope_dev* rope,
                         const uint8_t* k_codes, const int32_t* k_exps,
                         const uint8_t* v_codes, const int32_t* v_exps, int32_t n_layers,
                         int32_t row_begin, int32_t n_rows, void* k_cache, void* v_cache,
                         int64_t layer_stride_elems, int32_t T, const int32_t* chunk_offsets,
                         int32_t n_chunks, int32_t shift, void* stream);

/* One layer's weights as 8-bit E4M3 codes with one power-of-two exponent
 * per output row (cb_quantize_fp8 over the rows of each [out][in] matrix):
 *  w_qkv [q_dim + 2 kv_dim][d]: the rows of W_q, then W_k, then W_v;
 *  w_o [d][q_dim]; w_gu [2 ffn][d]: the rows of W_gate, then W_up;
 *  w_down [d][ffn]; e_* int32 [rows]; attn_norm, mlp_norm fp32 [d].
 * Device pointers, codes 16-byte aligned. */
typedef struct {
  const float* attn_norm;
  const uint8_t* w_qkv;
  const int32_t* e_qkv;
  const uint8_t* w_o;
  const int32_t* e_o;
  const float* mlp_norm;
  const uint8_t* w_gu;
  const int32_t* e_gu;
  const uint8_t* w_down;
  const int32_t* e_down;
} cb_layer_weights_fp8;

/* Bytes of workspace cb_blend_layer_fp8 needs (cb_workspace_size plus the
 * activation codes and the fp32 products).  0 on invalid cfg. */
size_t cb_workspace_size_fp8(const cb_layer_config* cfg, int32_t T, int32_t m_max);

/* cb_blend_layer with 8-bit projections, the way the paper serves its larger
 * models (section 7, 8-bit weights): every projection's input rows (the normalised x, the
 * attention output, the normalised h, u; stored in bf16 as in cb_blend_layer) are quantized
 * per row to E4M3 (as cb_quantize_fp8) and multiplied with the 8-bit weights
 * on the fp8 matrix cores (as cb_gemm_fp8, fp32 products); RoPE, the K
 * deviation, the scatter, the top-k, the attention, the residuals, the
 * RMSNorms and SwiGLU are those of cb_blend_layer.  cfg->dtype must be
 * CB_BF16 (CB_ERR_UNSUPPORTED) and d_model, q_dim and ffn_dim multiples of
 * 16 (CB_ERR_SHAPE).  Arguments, results and other errors as cb_blend_layer;
 * workspace >= cb_workspace_size_fp8(cfg, T, m_in). */
cb_status cb_blend_layer_fp8(const cb_layer_config* cfg, const cb_layer_weights_fp8* w,
                             const cb_rope_dev* rope, void* k_cache, void* v_cache, int32_t T,
                             int32_t n_ctx, int32_t first_chunk_len, const int32_t* s_in,
                             int32_t m_in, const void* hidden_in, const int32_t* in_rows,
                             int32_t k_out, void* hidden_out, float* dev_out, int32_t* s_out,
                             int32_t* m_out_host, void* ws, size_t ws_bytes, void* stream);

/* cb_blend_stack with the chunk KV of every layer loaded from 8-bit host
 * copies: k_src, v_src host uint8 [n_layers][T][n_kv][hd] and k_src_exp,
 * v_src_exp host int32 [n_layers][T][n_kv] (allocate with hipHostMalloc for
 * asynchronous copies).  Layer l's codes are copied into a device staging
 * slot in the workspace and expanded into its caches on copy_stream
 * (cb_kv_from_fp8 over all T rows, re-aligning the keys when shift != 0);
 * layer l's recompute waits for that expansion only.  Every other argument,
 * the results and the errors are those of cb_blend_stack; the result equals
 * cb_blend_stack run on caches holding the expanded values. */
cb_status cb_blend_stack_kv8(const cb_layer_config* cfg, int32_t n_layers,
                             const cb_layer_weights* layers, const cb_rope_dev* rope,
                             void* k_caches, void* v_caches, int64_t layer_stride_elems,
                             const uint8_t* k_src, const int32_t* k_src_exp,
                             const uint8_t* v_src, const int32_t* v_src_exp, int32_t T,
                             const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift,
                             const void* x_first, const int32_t* ks, int32_t* s_out_all,
                             float* dev_all, void* hidden_out, int32_t* m_rows_host, void* ws,
                             size_t ws_bytes, void* stream, void* copy_stream);

#ifdef __cplusplus
}
#endif

#endif /* CACHEBLEND_H */
