// Internal declarations shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cacheblend.h"

namespace cb {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float rnd(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float rnd(float v) { return bf2f(f2bf(v)); }
};

// Load / store 8 consecutive elements (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f2bf(v[2 * j]) | ((uint32_t)f2bf(v[2 * j + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Composite row map: r = i; r = m1[r] if m1; r = m2[r] if m2.
__device__ __forceinline__ int map_row(int i, const int* m1, const int* m2) {
  int r = m1 ? m1[i] : i;
  return m2 ? m2[r] : r;
}

// ---------------------------------------------------------------------------
// Kernel timing hooks (host side).  When profiling is on, every launch below
// is bracketed by hipEvents recorded on its stream.
// ---------------------------------------------------------------------------
struct LaunchScope {
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  int slot;
  hipStream_t stream;
};

// ---------------------------------------------------------------------------
// Launchers (host).  All return hipSuccess or the launch error.
// ---------------------------------------------------------------------------

// Several requests in one launch (the batched fusor): the rows of request r
// are rows row_off[r] .. row_off[r+1]-1 of the launch, and each request has
// its own K/V cache and length.  n = 0: one request, described by the
// launch's scalar fields.  Read with a row (or tile) index in every kernel
// that needs the cache of a row.
constexpr int kMaxReq = 16;
struct ReqTable {
  int n;
  int row_off[kMaxReq + 1];
  int tile_off[kMaxReq + 1];   // attention: first row tile of request r
  void* k[kMaxReq];
  void* v[kMaxReq];
  int T[kMaxReq];
  int lo[kMaxReq], hi[kMaxReq];   // QKV: deviation for cache rows in [lo, hi)
};

// Cache policy bits of the GEMMs' direct-to-LDS operand loads.  The weight
// rows are read once per launch (each by the few workgroups of one output
// column block, close together in time), so they are loaded non-temporal
// (bit 1, nt), which leaves the caches to the activation rows that every
// output column block reads again and to the split-K partials that the
// finishing kernels read next (measured: the same L2 fetch bytes, a faster
// step, and the finishing kernels faster too, i.e. the memory-side Infinity
// Cache keeps more of those).  The activation rows use the default policy.
#ifndef CB_W_AUX
#define CB_W_AUX 2
#endif
#ifndef CB_A_AUX
#define CB_A_AUX 0
#endif

// s_waitcnt vmcnt(n) lgkmcnt(0): this wave's LDS DMA up to the n most recent
// loads has landed and its LDS reads have returned.
#define CB_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0070)
// Workgroup barrier without a memory fence (a fence would drain the DMA ring);
// the empty asm statements keep the compiler from moving LDS accesses across it.
#define CB_BARRIER()                  \
  do {                                \
    asm volatile("" ::: "memory");    \
    __builtin_amdgcn_s_barrier();     \
    asm volatile("" ::: "memory");    \
  } while (0)

typedef __attribute__((address_space(3))) void lds_void;

// SwiGLU gate: silu(g) = g / (1 + e^-g), with the hardware base-2 exponent
// and reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each); e^-g overflowing to
// infinity gives -0 for large negative g.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Buffer resource over `bytes` bytes at p (gfx9 layout: raw buffer, no
// stride); loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// request of row `row` (rows of empty requests are skipped)
__device__ __forceinline__ int req_of_row(const ReqTable& t, int row) {
  int r = 0;
  while (r + 1 < t.n && t.row_off[r + 1] <= row) ++r;
  return r;
}

struct RopeShiftArgs {
  void* k_cache;
  int64_t layer_stride;
  int n_layers;
  int T;
  int kv_dim;     // n_kv * hd
  int hd;
  const float* cos;
  const float* sin;
  const int32_t* offsets;  // host, n_chunks + 1
  int n_chunks;
};
hipError_t launch_rope_shift(int dtype, const RopeShiftArgs& a, hipStream_t s);

// Chunk offsets as kernel arguments (at most kMaxChunks chunks).
constexpr int kMaxChunks = 256;
struct ChunkOffsets {
  int32_t o[kMaxChunks + 1];
};

// Re-alignment offset of cache row r >= o[1]: o[c] of the chunk c >= 1 that
// holds it (the largest c in [1, n_chunks - 1] with o[c] <= r).
__device__ __forceinline__ int chunk_delta(const ChunkOffsets& offs, int n_chunks, int r) {
  int lo = 1, hi = n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs.o[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return offs.o[lo];
}

// The same offset found by a scan whose loads do not depend on r: with the
// offsets in kernel arguments every load is uniform (scalar), so a thread
// does not wait on a chain of dependent vector loads.
__device__ __forceinline__ int chunk_delta_scan(const ChunkOffsets& offs, int n_chunks, int r) {
  int delta = offs.o[1];
  for (int c = 2; c < n_chunks; ++c) {
    const int oc = offs.o[c];
    delta = oc <= r ? oc : delta;
  }
  return delta;
}

// Rotation of 4 consecutive (even, odd) pairs by the angles whose cos / sin
// are cs[0..3] / sn[0..3]: two rounded products and one rounded sum per
// output, never contracted into fused multiply-adds, so every kernel that
// re-aligns a key gets the same bits.
__device__ __forceinline__ void rope_rotate8(const float v[8], const float* cs, const float* sn, float o[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = v[2 * j], b = v[2 * j + 1], c = cs[j], s = sn[j];
    o[2 * j] = a * c - b * s;
    o[2 * j + 1] = a * s + b * c;
  }
}

// One layer's re-alignment run inside the launch of its QKV projection
// (bf16, no split-K): the first n_wg workgroups of that launch rotate the
// keys of rows [row0, row1) (chunks >= 1) that the call does not recompute
// (not in s_in), and the projection's deviation epilogue compares each new
// key with its cached key re-aligned in registers.  The cache then ends up
// as after a separate cb_rope_shift followed by the layer, bit for bit.
struct ShiftFuse {
  int n_wg;
  int row0, row1;
  int n_chunks;
  int kv_dim, hd;
  void* k;                 // the layer's K cache [T][kv_dim]
  const float* cos;        // [n_pos][hd / 2]
  const float* sin;
  const int32_t* s_in;     // rows the call recomputes (device)
  int m_in;
  ChunkOffsets offs;
};

// Expansion of 8-bit stored K/V (E4M3 codes, one power-of-two exponent per
// (row, KV head)) into the cache, keys re-aligned when shift != 0.
constexpr int kMaxShiftChunks = 256;
struct KvExpandArgs {
  const uint8_t* k_codes;   // [n_layers][n_rows][kv_dim]
  const int32_t* k_exps;    // [n_layers][n_rows][n_kv]
  const uint8_t* v_codes;
  const int32_t* v_exps;
  void* k_cache;            // layer l, row r at l * layer_stride + r * kv_dim
  void* v_cache;
  int64_t layer_stride;
  int n_layers;
  int row0;                 // first cache row written
  int n_rows;
  int kv_dim, n_kv, hd;     // hd a multiple of 16
  const float* cos;         // RoPE tables (when shift)
  const float* sin;
  int n_chunks;
  int shift;
};
hipError_t launch_kv_expand(int dtype, const KvExpandArgs& a, const int32_t* offsets, hipStream_t s);

// RMSNorm of gathered rows: out[i] = x[map(i)] / sqrt(mean(x^2) + eps) * g.
// x_f32 selects an fp32 input regardless of the storage dtype.
// out[i] = start + i for i < n (the row list of a stack's first layer)
hipError_t launch_iota(int* out, int n, int start, hipStream_t s);

// packed_out: write the rows in the step-major layout of act_packed_index
// (bf16 output, d a multiple of 32)
hipError_t launch_rmsnorm(int dtype, bool x_f32, const void* x, int n_src, const int* m1, const int* m2,
                          const float* g, void* out, int rows, int d, float eps, hipStream_t s,
                          bool packed_out = false);

// Deviation of candidate rows, then top-k.  See select.hip.
struct SelectArgs {
  const float* dev_part;   // [n_parts][ld_part] partial sums, or NULL
  int n_parts;
  int ld_part;
  float* dev;              // [m_in] full deviation (written from the partials, or read)
  int n_cand;              // candidates are entries 0 .. n_cand-1
  int m_in;                // entries n_cand .. m_in-1 are always kept (query rows)
  int k;                   // candidates to keep
  const int* ids_in;       // token ids of the entries, NULL = identity
  int* sel;                // [m_out] kept entry positions, ascending (may be NULL)
  int* ids_out;            // [m_out] kept token ids (may be NULL)
  uint32_t* scratch;       // >= 16 words
  // several requests: workgroup g selects within entries in_off .. in_off+m_in-1
  // (the first n_cand are its candidates) and writes from out_off; sel values
  // are positions in the whole entry list
  int n_seg;               // 0 = one segment given by the fields above
  struct Seg {
    int in_off, m_in, n_cand, k, out_off;
  } seg[kMaxReq];
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// dev[i] = sum over kv_dim of (k_new[i] - k_ref[rows[i]])^2.
hipError_t launch_kdev(int dtype, const void* k_new, const void* k_ref, const int* rows, int n,
                       int kv_dim, int T, float* dev, hipStream_t s);

// ---------------------------------------------------------------------------
// GEMM: C[M][N] = A[M][K] * B[N][K]^T with fused epilogues.
// ---------------------------------------------------------------------------
struct BOperand {
  // mode 0: rows [0, n1) from p0, [n1, n2) from p1, [n2, N) from p2.
  // mode 1 (gated pair): output tile columns [0, BN/2) are rows of p0
  //   (features tile*BN/2 + j) and [BN/2, BN) the same rows of p1; n_feat
  //   features in total.
  int mode;
  const void* p0;
  const void* p1;
  const void* p2;
  int n1, n2;
  int n_feat;
  // mode 1 only, optional: the pair already in the large kernel's streaming
  // order (see launch_pack_gateup); p0/p1 are then not read
  const void* packed;
};
// The gate/up operand in the order the gated kernel streams it: for each
// tile of kGateupTile/2 features and each kGateupStep-element K step, the
// tile's gate rows then the same up rows, kGateupStep elements each, as one
// contiguous block; rows past n_feat and K past K are zero.
#ifndef CB_W4_BN
#define CB_W4_BN 224
#endif
constexpr int kGateupTile = CB_W4_BN, kGateupStep = 32;
__host__ __device__ inline size_t pack_gateup_bytes(int n_feat, int K) {
  const size_t tiles = (size_t)(n_feat + kGateupTile / 2 - 1) / (kGateupTile / 2);
  const size_t nk = (size_t)(K + kGateupStep - 1) / kGateupStep;
  return tiles * nk * kGateupTile * kGateupStep * 2;
}
hipError_t launch_pack_gateup(const void* w_gate, const void* w_up, int n_feat, int K, void* packed, hipStream_t s);

enum EpiKind { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_STORE = 3 };

struct EpiParams {
  int kind;
  // QKV
  int q_dim, kv_dim, hd;
  const int* rows;        // cache row of GEMM row i (NULL = i)
  int pos0;               // RoPE position = cache row + pos0
  int dev_lo, dev_hi;     // deviation for cache rows in [dev_lo, dev_hi)
  const float* cos;
  const float* sin;
  void* q_out;            // [M][q_dim]
  void* k_cache;          // [T][kv_dim]
  void* v_cache;
  int T;
  float* dev_part;        // [n_k_tiles][M] or NULL
  int k_tile0;            // first N tile intersecting the K columns
  ReqTable req;           // several requests: caches, T and deviation rows per GEMM row range
  // RESID: out[i][c] = resid[map(i)][c] + acc
  const void* resid;
  int resid_f32;
  const int* rmap1;
  const int* rmap2;
  void* out;
  int out_f32;
  int ld_out;
};

struct GemmArgs {
  const void* A;
  int M, N, K;
  BOperand B;
  EpiParams epi;
  int splits;             // split-K factor (bf16 only)
  float* part;            // [splits][M][n_tiles*BN] fp32 partials when splits > 1
  // RMSNorm folded into the bf16 QKV projection (a_norm != 0, splits == 1):
  // row i of A is row a_rows[i] (NULL = i) of an un-normalised [a_src_rows][K]
  // buffer; the product of row i is scaled by 1 / sqrt(mean(A_i^2) + a_eps)
  // before the epilogue (the RMSNorm gain is folded into B).
  int a_norm;
  const int* a_rows;
  int a_src_rows;
  float a_eps;
  // host-side: when set (QKV, bf16, no split-K), launch_gemm runs the
  // re-alignment it describes in the same launch
  const ShiftFuse* shift;
  // gate/up only: A is in the step-major layout of act_packed_index (see
  // gemm_gateup_packed_a)
  int a_packed;
};

// Step-major layout of a bf16 activation matrix [rows][d] (d a multiple of
// 32) for the gate/up projection: 256-row tiles, each a run of 32-column
// steps, each step the tile's 256 rows x 32 columns row by row (16 KB), so
// that one K step of a row tile is contiguous.  Index of element (i, c);
// act_packed_rows(rows) rows are stored (the last tile padded).
__host__ __device__ inline int64_t act_packed_index(int i, int c, int d) {
  return (((int64_t)(i >> 8) * (d >> 5) + (c >> 5)) * 256 + (i & 255)) * 32 + (c & 31);
}
__host__ __device__ inline int act_packed_rows(int rows) { return (rows + 255) / 256 * 256; }
// whether the bf16 gate/up projection over K = d takes its A operand in the
// step-major layout (then the MLP RMSNorm writes it so)
bool gemm_gateup_packed_a(int dtype, int K);

int gemm_bn(int dtype);                               // N tile width
int gemm_splits(int dtype, int N_tiles, int K);       // split-K choice (independent of M)
int gemm_n_tiles(int dtype, const BOperand& B, int N);
hipError_t launch_gemm(int dtype, const GemmArgs& g, hipStream_t s);
// whether launch_gemm runs g.shift inside the launch (otherwise the caller
// shifts first)
bool gemm_fuses_shift(int dtype, const GemmArgs& g);
// The epilogue of g.epi.kind (QKV, RESID or STORE; bf16 cache) applied to a
// product already in g.part (g.splits fp32 slices of row stride
// epilogue_ld(g.N)), e.g. one written by the fp8 GEMM.
hipError_t launch_epilogue_only(const GemmArgs& g, hipStream_t s);
int epilogue_ld(int N);
// ... the RESID epilogue into fp32 h followed by the RMSNorm of h into hn
hipError_t launch_resid_norm_only(const GemmArgs& g, const float* gain, float eps, void* hn, hipStream_t s,
                                  bool hn_packed = false);
// A residual projection into fp32 rows (epi.out) followed by the RMSNorm of
// those rows into hn (the cache dtype), fused after split-K when possible.
hipError_t launch_gemm_resid_norm(int dtype, const GemmArgs& g, const float* gain, float eps, void* hn,
                                  hipStream_t s, bool hn_packed = false);

// ---------------------------------------------------------------------------
// Attention of selected rows over the cache.
// ---------------------------------------------------------------------------
// fp8 E4M3 operands with one power-of-two scale per row:
// C[i][j] = sum_k A[i][k] B[j][k] * 2^(a_exp[i] + b_exp[j]); A [M][K], B [N][K]
// row-major codes; C [M][ldc] in the output dtype.
struct Fp8GemmArgs {
  const uint8_t* A;
  const int* a_exp;
  const uint8_t* B;
  const int* b_exp;
  void* C;
  int M, N, K, ldc;
  int splits;     // split-K factor (fp32 partials in part, summed in order)
  float* part;    // [splits][M][N]
  int keep_parts; // splits > 1: leave the partials in part for the caller to sum
  int gated_F;    // > 0: B = [W_gate; W_up] (2 gated_F rows) and C = silu(A W_gate^T) * (A W_up^T), bf16 [M][ldc]
};
int fp8_splits(int N, int K);
hipError_t launch_quantize_rows(int src_dtype, const void* x, int rows, int cols, uint8_t* q, int* ex,
                                hipStream_t s);
hipError_t launch_gemm_fp8(const Fp8GemmArgs& g, int out_dtype, hipStream_t s);

constexpr int kAttnRowTile = 32;   // kept rows per attention workgroup (one row tile)

struct AttnArgs {
  const void* Q;          // [*][n_q*hd]; row qmap[i] (NULL = i) holds query i
  const int* qmap;
  const int* qpos;        // query i attends cache rows 0 .. qpos[i] (NULL = i)
  const void* K;          // [T][n_kv*hd]
  const void* V;
  void* O;                // [m][n_q*hd]
  int m, T, n_q, n_kv, hd;
  int key_split;          // 0: one pass over all keys; else keys split at multiples of this
  bf16_t* o_part;         // [T / key_split][m][n_q][hd] unnormalised partials, bf16 (key_split > 0)
  float* ml_part;         // [T / key_split][m][n_q][2] running max (log2 units) and sum
  ReqTable req;           // several requests: row ranges, row tiles, K/V and T per request (T = max)
  // When a layer keeps every recomputed row, no selection kernel runs and the
  // bf16 attention writes its outputs instead (fin_ids_out != NULL):
  // fin_ids_out[i] = fin_ids_in[i], fin_dev[i] = the sum of the fin_n_parts
  // deviation partials in order (NaN for i >= fin_n_cand), i < m.
  const int* fin_ids_in;
  int* fin_ids_out;
  const float* fin_dev_part;
  float* fin_dev;
  int fin_n_parts, fin_ld_part, fin_n_cand;
};
// Key-split length used for m query rows over T keys (0 = none): a multiple
// of 64, at least 512; chosen from the row, head and key counts only.
// attn_part_rows bounds the m for which it is non-zero.
int attn_key_split(int dtype, int m, int n_kv, int T);
size_t attn_part_rows(int n_q, int n_kv);
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s);

// Deviation analytics (diagnostics): part >= m * n_q * 2 doubles, out device [2].
hipError_t launch_attention_deviation(int dtype, int m, int n_q, int n_kv, int hd, const void* qa, const void* ka,
                                      const void* qb, const void* kb, int T, const int* last_key, double* part,
                                      double* out, hipStream_t s);
// ranks >= 2n doubles; out device [1]
hipError_t launch_spearman(const float* x, const float* y, int n, double* ranks, double* out, hipStream_t s);
// contrib >= n doubles; out device [1]
hipError_t launch_top_share(const float* x, int n, int k, double* contrib, double* out, hipStream_t s);

// W_qkv [n_rows][K] bf16 = [W_q; W_k; W_v] with column k scaled by gain[k]
// (rounded to bf16), the B operand of the QKV projection with the RMSNorm
// folded in.
hipError_t launch_fold_qkv(const void* w_q, const void* w_k, const void* w_v, int n_q_rows, int n_kv_rows, int K,
                           const float* gain, void* out, hipStream_t s);

// Streaming copy of bytes / 16 16-byte units (bytes % 16 == 0, both 16-byte aligned).
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace cb
