// C ABI of the fusor: argument checks, workspace layout and the launch
// sequence of one layer on the caller's stream.
//
// cb_blend_layer follows CacheBlend (arXiv 2405.16444) section 4.2, Figure
// 5b, with the HKVD selection of section 4.3:
//   1. mask: gather the selected rows' inputs and apply the attention RMSNorm
//   2. Q/K/V of those rows only; RoPE at their absolute positions; the K
//      deviation against the cached row is summed before the new K/V replace
//      the cached entries (expansion with the reused entries of other rows)
//   3. keep the top-k rows by deviation plus the query rows
//   4. attention of the kept rows over the blended cache
//   5. output projection + residual, RMSNorm, SwiGLU MLP + residual
// Every step is a kernel enqueued on the caller's stream; the host never
// waits on the device.
#include <math.h>

#include <cmath>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "cb_internal.h"

namespace cb {

// ---------------------------------------------------------------------------
// per-thread state: last HIP error, optional kernel timing
// ---------------------------------------------------------------------------
namespace {

thread_local int32_t t_last_hip = 0;
thread_local bool t_validate = false;

struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
thread_local bool t_prof = false;
thread_local std::vector<ProfRec> t_recs;
thread_local std::vector<hipEvent_t> t_pool;

hipEvent_t pool_get() {
  if (!t_pool.empty()) {
    hipEvent_t e = t_pool.back();
    t_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

cb_status hip_status(hipError_t e) {
  if (e == hipSuccess) return CB_OK;
  t_last_hip = (int32_t)e;
  return CB_ERR_HIP;
}

}  // namespace

LaunchScope::LaunchScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  if (!t_prof) return;
  ProfRec r{name, pool_get(), pool_get()};
  if (!r.a || !r.b) return;
  (void)hipEventRecord(r.a, s);
  t_recs.push_back(r);
  slot = (int)t_recs.size() - 1;
}

LaunchScope::~LaunchScope() {
  if (slot >= 0) (void)hipEventRecord(t_recs[slot].b, stream);
}

// ---------------------------------------------------------------------------
// validation and workspace
// ---------------------------------------------------------------------------
namespace {

cb_status check_cfg(const cb_layer_config* c) {
  if (!c) return CB_ERR_ARG;
  if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->ffn_dim <= 0)
    return CB_ERR_ARG;
  if (c->dtype != CB_F32 && c->dtype != CB_BF16) return CB_ERR_ARG;
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return CB_ERR_ARG;
  if (c->n_q_heads % c->n_kv_heads) return CB_ERR_SHAPE;
  if (c->head_dim % 8 || c->d_model % 8 || c->ffn_dim % 8) return CB_ERR_SHAPE;
  if (c->dtype == CB_BF16) {
    if (c->head_dim != 64 && c->head_dim != 128) return CB_ERR_UNSUPPORTED;
    const int g = c->n_q_heads / c->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return CB_ERR_UNSUPPORTED;
  } else if (c->head_dim > 256) {
    return CB_ERR_UNSUPPORTED;
  }
  return CB_OK;
}

constexpr int kF32MaxT = 8192;  // fp32 attention keeps a row's scores in LDS

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
  int d, q_dim, kv_dim, n_kv, hd, F, b, bn;
  explicit Dims(const cb_layer_config& c)
      : d(c.d_model), q_dim(c.n_q_heads * c.head_dim), kv_dim(c.n_kv_heads * c.head_dim), n_kv(c.n_kv_heads),
        hd(c.head_dim), F(c.ffn_dim), b(c.dtype == CB_BF16 ? 2 : 4), bn(gemm_bn(c.dtype)) {}
  int n_qkv() const { return q_dim + 2 * kv_dim; }
  int k_tile0() const { return q_dim / bn; }
  int n_k_tiles() const { return (q_dim + kv_dim - 1) / bn - k_tile0() + 1; }
};

struct Ws {
  size_t xn, q, devp, dev, sel, o, h, hn, u, part, o_part, ml_part, scratch, total;
};

BOperand b_single(const void* p, int n) {
  BOperand B{};
  B.mode = 0;
  B.p0 = B.p1 = B.p2 = p;
  B.n1 = B.n2 = n;
  B.n_feat = n;
  return B;
}

size_t part_floats(int dtype, const Dims& D, int m) {
  // largest split-K partial buffer over the four projections
  size_t best = 0;
  auto consider = [&](const BOperand& B, int N, int K) {
    const int nt = gemm_n_tiles(dtype, B, N);
    const int sp = gemm_splits(dtype, nt, K);
    if (sp > 1) best = std::max(best, (size_t)sp * m * nt * D.bn);
  };
  BOperand qkv = b_single(nullptr, D.n_qkv());
  consider(qkv, D.n_qkv(), D.d);
  consider(b_single(nullptr, D.d), D.d, D.q_dim);
  BOperand gu{};
  gu.mode = 1;
  gu.n_feat = D.F;
  consider(gu, 0, D.d);
  consider(b_single(nullptr, D.d), D.d, D.F);
  return best;
}

// Workspace for up to m rows over a cache of T rows.
Ws layout(const cb_layer_config& c, int m, int T) {
  const Dims D(c);
  Ws w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t M = (size_t)std::max(m, 1);
  w.xn = take(M * D.d * D.b);
  w.q = take(M * D.q_dim * D.b);
  w.devp = take((size_t)D.n_k_tiles() * M * 4);
  w.dev = take(M * 4);
  w.sel = take(M * 4);
  w.o = take(M * D.q_dim * D.b);
  w.h = take(M * D.d * 4);
  w.hn = take((size_t)act_packed_rows((int)M) * D.d * D.b);   // row-major or step-major (gate/up input)
  w.u = take(M * D.F * D.b);
  w.part = take(part_floats(c.dtype, D, (int)M) * 4);
  // attention key-split partials: only for row counts that use the split
  const size_t arows = std::min(M, attn_part_rows(c.n_q_heads, c.n_kv_heads));
  const size_t nsplit = c.dtype == CB_BF16 ? (size_t)(std::max(T, 1) + 511) / 512 : 0;
  w.o_part = take(nsplit * arows * D.q_dim * 2);   // bf16 partials
  w.ml_part = take(nsplit * arows * c.n_q_heads * 8);
  w.scratch = take(256);
  w.total = off;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

cb_status check_rope(const cb_layer_config* c, const cb_rope_dev* r, int need) {
  if (!r || !r->cos || !r->sin || !aligned16(r->cos) || !aligned16(r->sin)) return CB_ERR_ARG;
  // a table is only valid for the base and head size it was built with
  if (r->head_dim != c->head_dim || r->rope_theta != c->rope_theta) return CB_ERR_ARG;
  if (r->n_pos < need) return CB_ERR_SHAPE;
  return CB_OK;
}

cb_status check_weights(const cb_layer_weights* w) {
  if (!w) return CB_ERR_ARG;
  const void* p[9] = {w->attn_norm, w->w_q, w->w_k, w->w_v, w->w_o, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  for (const void* x : p)
    if (!x || !aligned16(x)) return CB_ERR_ARG;
  if (w->w_gateup_packed && !aligned16(w->w_gateup_packed)) return CB_ERR_ARG;
  if (w->w_qkv_folded && !aligned16(w->w_qkv_folded)) return CB_ERR_ARG;
  return CB_OK;
}

// Extra workspace of the 8-bit layer, after the bf16 layout of the same size:
// activation codes and row exponents, the fp32 product of one projection
// (QKV, O, down; the gate/up product never leaves its kernel) and the fp8
// GEMM's split-K partials.
struct Fp8Ws {
  size_t codes, exps, prod, part, total;
};

size_t fp8_part_bytes(int M, int N, int K) {
  const int sp = fp8_splits(N, K);
  return sp > 1 ? (size_t)sp * M * N * 4 : 0;
}

Fp8Ws layout_fp8(const cb_layer_config& c, int m, size_t base) {
  const Dims D(c);
  const size_t M = (size_t)std::max(m, 1);
  Fp8Ws w{};
  size_t off = base;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.codes = take(M * std::max(std::max(D.d, D.q_dim), D.F));
  w.exps = take(M * 4);
  w.prod = take(M * std::max((size_t)epilogue_ld(D.n_qkv()), (size_t)epilogue_ld(D.d)) * 4);
  w.part = take(std::max(std::max(fp8_part_bytes((int)M, D.n_qkv(), D.d), fp8_part_bytes((int)M, D.d, D.q_dim)),
                         std::max(fp8_part_bytes((int)M, 2 * D.F, D.d), fp8_part_bytes((int)M, D.d, D.F))));
  w.total = off;
  return w;
}

// Rows of A (bf16 [M][K]) quantized to E4M3 per row, times the 8-bit
// weights [N][K], scaled by both row exponents, in fp32: in C (row stride
// ldc) or, when K is split and ldc == N, left as the split partials, which
// the epilogue kernels sum in split order.  *out / *splits say which.
cb_status proj_fp8(const void* A, int M, int K, const uint8_t* w, const int32_t* we, int N, float* C, int ldc,
                   const Fp8Ws& F8, void* ws, hipStream_t s, float** out, int* splits) {
  uint8_t* codes = at<uint8_t>(ws, F8.codes);
  int* exps = at<int>(ws, F8.exps);
  cb_status st = hip_status(launch_quantize_rows(CB_BF16, A, M, K, codes, exps, s));
  if (st) return st;
  Fp8GemmArgs g{};
  g.A = codes;
  g.a_exp = exps;
  g.B = w;
  g.b_exp = we;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.splits = fp8_splits(N, K);
  g.part = at<float>(ws, F8.part);
  g.keep_parts = g.splits > 1 && ldc == N;
  *out = g.keep_parts ? g.part : C;
  *splits = g.keep_parts ? g.splits : 1;
  return hip_status(launch_gemm_fp8(g, CB_F32, s));
}

// u = silu(x W_gate^T) * (x W_up^T) (bf16 [M][F]) with 8-bit x rows and
// weights w_gu = [W_gate; W_up], SwiGLU in the GEMM's epilogue
cb_status proj_fp8_gated(const void* A, int M, int K, const uint8_t* w, const int32_t* we, int F, void* u,
                         const Fp8Ws& F8, void* ws, hipStream_t s) {
  uint8_t* codes = at<uint8_t>(ws, F8.codes);
  int* exps = at<int>(ws, F8.exps);
  cb_status st = hip_status(launch_quantize_rows(CB_BF16, A, M, K, codes, exps, s));
  if (st) return st;
  Fp8GemmArgs g{};
  g.A = codes;
  g.a_exp = exps;
  g.B = w;
  g.b_exp = we;
  g.C = u;
  g.M = M;
  g.N = 2 * F;
  g.K = K;
  g.ldc = F;
  g.splits = 1;
  g.gated_F = F;
  return hip_status(launch_gemm_fp8(g, CB_BF16, s));
}

// The part of a layer after attention: O projection + residual, RMSNorm,
// SwiGLU MLP, down projection + residual.  resid rows: map(i) = m2[m1[i]].
cb_status layer_tail(const cb_layer_config& c, const cb_layer_weights& w, const Ws& L, void* ws, int m_out,
                     const void* hidden_in, int n_resid, const int* m1, const int* m2, void* hidden_out,
                     hipStream_t s, const cb_layer_weights_fp8* w8 = nullptr, const Fp8Ws* F8 = nullptr) {
  const Dims D(c);
  const int dt = c.dtype;
  // O projection + residual -> h (fp32)
  GemmArgs g{};
  g.A = at<void>(ws, L.o);
  g.M = m_out;
  g.N = D.d;
  g.K = D.q_dim;
  g.B = b_single(w.w_o, D.d);
  g.epi.kind = EPI_RESID;
  g.epi.resid = hidden_in;
  g.epi.resid_f32 = 0;
  g.epi.rmap1 = m1;
  g.epi.rmap2 = m2;
  g.epi.T = n_resid;
  g.epi.out = at<void>(ws, L.h);
  g.epi.out_f32 = 1;
  g.epi.ld_out = D.d;
  g.splits = gemm_splits(dt, gemm_n_tiles(dt, g.B, g.N), g.K);
  g.part = at<float>(ws, L.part);
  // ... and RMSNorm(h) -> hn, in the step-major layout when the bf16
  // gate/up projection reads it so
  const bool hn_packed = !w8 && gemm_gateup_packed_a(dt, D.d);
  cb_status st;
  if (w8) {
    st = proj_fp8(g.A, m_out, D.q_dim, w8->w_o, w8->e_o, D.d, at<float>(ws, F8->prod), epilogue_ld(D.d), *F8, ws,
                  s, &g.part, &g.splits);
    if (st) return st;
    st = hip_status(launch_resid_norm_only(g, (const float*)w.mlp_norm, c.rms_eps, at<void>(ws, L.hn), s));
  } else {
    st = hip_status(
        launch_gemm_resid_norm(dt, g, (const float*)w.mlp_norm, c.rms_eps, at<void>(ws, L.hn), s, hn_packed));
  }
  if (st) return st;
  // gate/up + SwiGLU -> u
  GemmArgs gu{};
  gu.A = at<void>(ws, L.hn);
  gu.M = m_out;
  gu.K = D.d;
  gu.B.mode = 1;
  gu.B.p0 = w.w_gate;
  gu.B.p1 = w.w_up;
  gu.B.p2 = w.w_up;
  gu.B.n_feat = D.F;
  gu.B.packed = dt == CB_BF16 ? w.w_gateup_packed : nullptr;
  gu.a_packed = hn_packed ? 1 : 0;
  gu.epi.kind = EPI_SWIGLU;
  gu.epi.out = at<void>(ws, L.u);
  gu.epi.ld_out = D.F;
  gu.splits = gemm_splits(dt, gemm_n_tiles(dt, gu.B, 0), gu.K);
  gu.part = at<float>(ws, L.part);
  if (w8) {
    st = proj_fp8_gated(gu.A, m_out, D.d, w8->w_gu, w8->e_gu, D.F, gu.epi.out, *F8, ws, s);
  } else {
    st = hip_status(launch_gemm(dt, gu, s));
  }
  if (st) return st;
  // down projection + residual (h) -> hidden_out
  GemmArgs gd{};
  gd.A = at<void>(ws, L.u);
  gd.M = m_out;
  gd.N = D.d;
  gd.K = D.F;
  gd.B = b_single(w.w_down, D.d);
  gd.epi.kind = EPI_RESID;
  gd.epi.resid = at<void>(ws, L.h);
  gd.epi.resid_f32 = 1;
  gd.epi.T = m_out;
  gd.epi.out = hidden_out;
  gd.epi.out_f32 = dt == CB_F32;
  gd.epi.ld_out = D.d;
  gd.splits = gemm_splits(dt, gemm_n_tiles(dt, gd.B, gd.N), gd.K);
  gd.part = at<float>(ws, L.part);
  if (w8) {
    st = proj_fp8(gd.A, m_out, D.F, w8->w_down, w8->e_down, D.d, at<float>(ws, F8->prod), epilogue_ld(D.d), *F8,
                  ws, s, &gd.part, &gd.splits);
    if (st) return st;
    return hip_status(launch_epilogue_only(gd, s));
  }
  return hip_status(launch_gemm(dt, gd, s));
}

// Fill the QKV projection arguments.
GemmArgs qkv_args(const cb_layer_config& c, const cb_layer_weights& w, const cb_rope_dev& rope, const Ws& L,
                  void* ws, int M) {
  const Dims D(c);
  GemmArgs g{};
  g.A = at<void>(ws, L.xn);
  g.M = M;
  g.N = D.n_qkv();
  g.K = D.d;
  g.B.mode = 0;
  g.B.p0 = w.w_q;
  g.B.p1 = w.w_k;
  g.B.p2 = w.w_v;
  g.B.n1 = D.q_dim;
  g.B.n2 = D.q_dim + D.kv_dim;
  g.B.n_feat = g.N;
  g.epi.kind = EPI_QKV;
  g.epi.q_dim = D.q_dim;
  g.epi.kv_dim = D.kv_dim;
  g.epi.hd = D.hd;
  g.epi.cos = rope.cos;
  g.epi.sin = rope.sin;
  g.epi.q_out = at<void>(ws, L.q);
  g.epi.k_tile0 = D.k_tile0();
  g.splits = gemm_splits(c.dtype, gemm_n_tiles(c.dtype, g.B, g.N), g.K);
  g.part = at<float>(ws, L.part);
  return g;
}

// The QKV projection's input.  With a folded weight copy (bf16, no split-K)
// the attention RMSNorm runs inside the projection: A is the raw rows
// (gathered through in_rows) and every row's product is scaled by its
// 1 / rms; otherwise a separate pass writes the normalised rows to xn.
cb_status qkv_input(const cb_layer_config& c, const cb_layer_weights& w, GemmArgs& g, const void* hidden,
                    int n_src, const int32_t* in_rows, int m, void* xn, bool allow_fold, hipStream_t s) {
  if (allow_fold && c.dtype == CB_BF16 && w.w_qkv_folded && g.splits == 1) {
    g.B.p0 = g.B.p1 = g.B.p2 = w.w_qkv_folded;
    g.B.n1 = g.B.n2 = g.N;
    g.A = hidden;
    g.a_norm = 1;
    g.a_rows = in_rows;
    g.a_src_rows = n_src;
    g.a_eps = c.rms_eps;
    return CB_OK;
  }
  return hip_status(launch_rmsnorm(c.dtype, false, hidden, n_src, nullptr, in_rows, (const float*)w.attn_norm, xn, m,
                                   c.d_model, c.rms_eps, s));
}

}  // namespace
}  // namespace cb

using namespace cb;

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------

extern "C" cb_status cb_rope_table(const cb_layer_config* cfg, int32_t pos_begin, int32_t n_pos, float* cos_out,
                                   float* sin_out) {
  if (!cfg || !cos_out || !sin_out || pos_begin < 0 || n_pos < 0) return CB_ERR_ARG;
  if (cfg->head_dim <= 0 || cfg->head_dim % 2 || !(cfg->rope_theta > 0.f)) return CB_ERR_ARG;
  const int half = cfg->head_dim / 2;
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
  for (int p = 0; p < n_pos; ++p) {
    for (int i = 0; i < half; ++i) {
      const double ang = (double)(pos_begin + p) * inv[i];
      cos_out[(size_t)p * half + i] = (float)cos(ang);
      sin_out[(size_t)p * half + i] = (float)sin(ang);
    }
  }
  return CB_OK;
}

extern "C" int32_t cb_num_selected(int32_t r_e4, int32_t n_ctx, int32_t n_cand) {
  if (r_e4 < 0 || n_ctx < 0 || n_cand < 0) return -1;
  const int64_t num = (int64_t)r_e4 * n_ctx;
  const int64_t k = (num + 9999) / 10000;  // ceil for num >= 0
  return (int32_t)std::min<int64_t>(k, n_cand);
}

extern "C" cb_status cb_filter_schedule(int32_t n_layers, int32_t r_first_e4, int32_t r_last_e4, int32_t n_ctx,
                                        int32_t n_cand, int32_t* k_out) {
  if (n_layers <= 0 || r_first_e4 < 0 || r_last_e4 < 0 || n_ctx < 0 || n_cand < 0 || !k_out) return CB_ERR_ARG;
  k_out[0] = n_cand;
  for (int l = 1; l < n_layers; ++l) {
    // r_l = r_first - (r_first - r_last) * (l-1)/(L-2), in units of 1e-4;
    // k = ceil(r_l * n_ctx / 1e4) computed exactly over the common denominator
    int64_t k;
    if (r_last_e4 == 0 || n_layers <= 2) {
      k = ((int64_t)r_first_e4 * n_ctx + 9999) / 10000;
    } else {
      const int64_t den = (int64_t)(n_layers - 2);
      const int64_t r_num = (int64_t)r_first_e4 * den - (int64_t)(r_first_e4 - r_last_e4) * (l - 1);
      const int64_t num = r_num * n_ctx;            // r_l * n_ctx * 1e4 * den
      const int64_t q = 10000 * den;
      k = num >= 0 ? (num + q - 1) / q : -((-num) / q);
    }
    k = std::min<int64_t>(k, n_cand);
    k = std::min<int64_t>(k, k_out[l - 1]);
    k_out[l] = (int32_t)std::max<int64_t>(k, 0);
  }
  return CB_OK;
}

extern "C" size_t cb_workspace_size(const cb_layer_config* cfg, int32_t T, int32_t m_max) {
  if (check_cfg(cfg) != CB_OK || T < 0 || m_max < 0) return 0;
  return layout(*cfg, std::max(T, m_max), T).total;
}

extern "C" const char* cb_status_string(cb_status s) {
  // a C caller may pass any int: read the bits as an int, never as an
  // out-of-range enumerator value
  int32_t v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case CB_OK: return "ok";
    case CB_ERR_ARG: return "invalid argument";
    case CB_ERR_SHAPE: return "inconsistent shape";
    case CB_ERR_INDEX: return "index out of range";
    case CB_ERR_WORKSPACE: return "workspace too small";
    case CB_ERR_UNSUPPORTED: return "unsupported shape for the gfx950 kernels";
    case CB_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" int32_t cb_last_hip_error(void) { return t_last_hip; }

extern "C" int32_t cb_set_validate(int32_t on) {
  const int32_t prev = t_validate ? 1 : 0;
  t_validate = on != 0;
  return prev;
}

namespace cb {
namespace {

// Copy n int32 (or float) values from the device after the stream's earlier
// work; false on a HIP failure (recorded).
template <typename T>
bool fetch(std::vector<T>& out, const T* dev, int n, hipStream_t s) {
  out.resize(n > 0 ? n : 0);
  if (n <= 0) return true;
  if (hip_status(hipMemcpyAsync(out.data(), dev, (size_t)n * sizeof(T), hipMemcpyDeviceToHost, s)) ||
      hip_status(hipStreamSynchronize(s)))
    return false;
  return true;
}

// s_in of one request: strictly ascending, within [first_chunk_len, T), and
// every query row n_ctx .. T-1 present (they are then its last T - n_ctx
// entries); in_rows within [0, n_src).
cb_status check_rows(const int32_t* s_in, int m_in, int T, int n_ctx, int first_chunk_len) {
  for (int i = 0; i < m_in; ++i) {
    if (s_in[i] < first_chunk_len || s_in[i] >= T) return CB_ERR_INDEX;
    if (i > 0 && s_in[i] <= s_in[i - 1]) return CB_ERR_INDEX;
  }
  const int q = T - n_ctx;
  for (int j = 0; j < q; ++j)
    if (s_in[m_in - q + j] != n_ctx + j) return CB_ERR_INDEX;
  return CB_OK;
}

cb_status validate_blend(const int32_t* s_in_d, int m_in, const int32_t* in_rows_d, int T, int n_ctx,
                         int first_chunk_len, hipStream_t s) {
  std::vector<int32_t> rows;
  if (!fetch(rows, s_in_d, m_in, s)) return CB_ERR_HIP;
  cb_status st = check_rows(rows.data(), m_in, T, n_ctx, first_chunk_len);
  if (st || !in_rows_d) return st;
  if (!fetch(rows, in_rows_d, m_in, s)) return CB_ERR_HIP;
  for (int i = 0; i < m_in; ++i)
    if (rows[i] < 0 || rows[i] >= T) return CB_ERR_INDEX;
  return CB_OK;
}

}  // namespace
}  // namespace cb

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------

extern "C" cb_status cb_profile_begin(void) {
  t_prof = true;
  return CB_OK;
}

extern "C" int32_t cb_profile_end(cb_kernel_stat* out, int32_t max_out) {
  t_prof = false;
  struct Acc {
    std::string name;
    int n;
    double tot, mn, mx;
  };
  std::vector<Acc> acc;
  int32_t bad = 0;
  for (auto& r : t_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      bad = 1;
    } else {
      auto it = std::find_if(acc.begin(), acc.end(), [&](const Acc& a) { return a.name == r.name; });
      if (it == acc.end()) acc.push_back(Acc{r.name, 1, ms, ms, ms});
      else {
        it->n += 1;
        it->tot += ms;
        it->mn = std::min(it->mn, (double)ms);
        it->mx = std::max(it->mx, (double)ms);
      }
    }
    t_pool.push_back(r.a);
    t_pool.push_back(r.b);
  }
  t_recs.clear();
  if (bad) return -1;
  const int n = (int)acc.size();
  for (int i = 0; i < n && i < max_out && out; ++i) {
    memset(&out[i], 0, sizeof(out[i]));
    strncpy(out[i].name, acc[i].name.c_str(), sizeof(out[i].name) - 1);
    out[i].launches = acc[i].n;
    out[i].total_ms = acc[i].tot;
    out[i].min_ms = acc[i].mn;
    out[i].max_ms = acc[i].mx;
  }
  return n;
}

// ---------------------------------------------------------------------------
// device calls
// ---------------------------------------------------------------------------

extern "C" cb_status cb_rope_shift(const cb_layer_config* cfg, const cb_rope_dev* rope, void* k_cache,
                                   int64_t layer_stride_elems, int32_t n_layers, int32_t T,
                                   const int32_t* chunk_offsets, int32_t n_chunks, void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (!k_cache || !chunk_offsets || n_layers < 0 || T < 0 || n_chunks < 1 || !aligned16(k_cache))
    return CB_ERR_ARG;
  if (n_chunks > 256) return CB_ERR_UNSUPPORTED;
  if (chunk_offsets[0] != 0) return CB_ERR_SHAPE;
  for (int c = 0; c < n_chunks; ++c)
    if (chunk_offsets[c + 1] < chunk_offsets[c]) return CB_ERR_SHAPE;
  if (chunk_offsets[n_chunks] > T) return CB_ERR_SHAPE;
  const Dims D(*cfg);
  if (n_layers > 1 && layer_stride_elems < (int64_t)T * D.kv_dim) return CB_ERR_SHAPE;
  if ((layer_stride_elems * D.b) % 16) return CB_ERR_ARG;
  st = check_rope(cfg, rope, n_chunks > 1 ? chunk_offsets[n_chunks - 1] + 1 : 0);
  if (st) return st;
  RopeShiftArgs a{};
  a.k_cache = k_cache;
  a.layer_stride = layer_stride_elems;
  a.n_layers = n_layers;
  a.T = T;
  a.kv_dim = D.kv_dim;
  a.hd = D.hd;
  a.cos = rope->cos;
  a.sin = rope->sin;
  a.offsets = chunk_offsets;
  a.n_chunks = n_chunks;
  return hip_status(launch_rope_shift(cfg->dtype, a, (hipStream_t)stream));
}

extern "C" cb_status cb_select_hkvd(const cb_layer_config* cfg, const void* k_new, const void* k_ref, int32_t T,
                                    const int32_t* cand_rows, int32_t n, int32_t k, float* dev, int32_t* sel_out,
                                    void* ws, size_t ws_bytes, void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (n < 0 || k < 0 || k > n || !dev || (k > 0 && !sel_out) || T < 0) return CB_ERR_ARG;
  if (k_new && (!k_ref || !aligned16(k_new) || !aligned16(k_ref))) return CB_ERR_ARG;
  if (!ws) return CB_ERR_ARG;
  if (ws_bytes < cb_workspace_size(cfg, T, n)) return CB_ERR_WORKSPACE;
  if (n == 0) return CB_OK;
  hipStream_t s = (hipStream_t)stream;
  const Dims D(*cfg);
  if (t_validate) {
    if (k_new) {
      std::vector<int32_t> rows;
      if (!cand_rows) return CB_ERR_ARG;
      if (!cb::fetch(rows, cand_rows, n, s)) return CB_ERR_HIP;
      for (int i = 0; i < n; ++i)
        if (rows[i] < 0 || rows[i] >= T) return CB_ERR_INDEX;
    } else {
      std::vector<float> d;
      if (!cb::fetch(d, (const float*)dev, n, s)) return CB_ERR_HIP;
      for (int i = 0; i < n; ++i)
        if (std::isnan(d[i])) return CB_ERR_ARG;
    }
  }
  if (k_new) {
    st = hip_status(launch_kdev(cfg->dtype, k_new, k_ref, cand_rows, n, D.kv_dim, T, dev, s));
    if (st) return st;
  }
  SelectArgs a{};
  a.dev = dev;
  a.n_cand = n;
  a.m_in = n;
  a.k = k;
  a.ids_in = cand_rows;
  a.ids_out = sel_out;
  return hip_status(launch_select(a, s));
}

namespace cb {
namespace {

// One blend layer with validated arguments (shared by cb_blend_layer and
// cb_blend_stack); m_in > 0.
cb_status blend_run(const cb_layer_config& c, const cb_layer_weights& w, const cb_rope_dev& rope, void* k_cache,
                    void* v_cache, int T, int n_ctx, int first_chunk_len, const int32_t* s_in, int m_in,
                    const void* hidden_in, const int32_t* in_rows, int k_out, void* hidden_out, float* dev_out,
                    int32_t* s_out, void* ws, hipStream_t s, const cb_layer_weights_fp8* w8 = nullptr,
                    const ShiftFuse* shift = nullptr) {
  const cb_layer_config* cfg = &c;
  const int n_query = T - n_ctx;
  const int n_cand = m_in - n_query;
  const int m_out = std::min(k_out, n_cand) + n_query;
  const Dims D(c);
  const Ws L = layout(c, std::max(T, m_in), T);
  const Fp8Ws F8 = layout_fp8(c, std::max(T, m_in), align256(L.total));
  const int dt = c.dtype;
  const int n_src = in_rows ? T : m_in;
  cb_status st;

  // 1-2. gather + attention RMSNorm, QKV + RoPE + deviation + K/V scatter
  GemmArgs g = qkv_args(c, w, rope, L, ws, m_in);
  st = qkv_input(c, w, g, hidden_in, n_src, in_rows, m_in, at<void>(ws, L.xn), w8 == nullptr, s);
  if (st) return st;
  g.epi.rows = s_in;
  g.epi.pos0 = 0;
  g.epi.dev_lo = first_chunk_len;
  g.epi.dev_hi = n_ctx;
  g.epi.k_cache = k_cache;
  g.epi.v_cache = v_cache;
  g.epi.T = T;
  g.epi.dev_part = at<float>(ws, L.devp);
  if (shift) {
    // the layer's re-alignment: inside the QKV launch where that kernel
    // allows it, else as its own launch before the projection reads the cache
    g.shift = shift;
    if (w8 || !gemm_fuses_shift(dt, g)) {
      g.shift = nullptr;
      RopeShiftArgs ra{};
      ra.k_cache = shift->k;
      ra.layer_stride = 0;
      ra.n_layers = 1;
      ra.T = T;
      ra.kv_dim = shift->kv_dim;
      ra.hd = shift->hd;
      ra.cos = shift->cos;
      ra.sin = shift->sin;
      ra.offsets = shift->offs.o;
      ra.n_chunks = shift->n_chunks;
      st = hip_status(launch_rope_shift(dt, ra, s));
      if (st) return st;
    }
  }
  if (w8) {
    st = proj_fp8(g.A, m_in, D.d, w8->w_qkv, w8->e_qkv, D.n_qkv(), at<float>(ws, F8.prod), epilogue_ld(D.n_qkv()),
                  F8, ws, s, &g.part, &g.splits);
    if (st) return st;
    st = hip_status(launch_epilogue_only(g, s));
  } else {
    st = hip_status(launch_gemm(dt, g, s));
  }
  if (st) return st;
  // 3. deviation sums + top-k + query rows.  A layer that keeps every
  // recomputed row (k_out >= candidates: the blend call at a fixed ratio)
  // needs no ranking; on the bf16 path the attention kernel then writes the
  // deviation sums and the kept ids, and the kept rows are the input rows.
  const bool keep_all = dt == CB_BF16 && k_out >= n_cand;
  SelectArgs sa{};
  sa.dev_part = at<float>(ws, L.devp);
  sa.n_parts = D.n_k_tiles();
  sa.ld_part = m_in;
  sa.dev = dev_out ? dev_out : at<float>(ws, L.dev);
  sa.n_cand = n_cand;
  sa.m_in = m_in;
  sa.k = k_out;
  sa.ids_in = s_in;
  sa.sel = at<int>(ws, L.sel);
  sa.ids_out = s_out;
  if (!keep_all) {
    st = hip_status(launch_select(sa, s));
    if (st) return st;
  }
  // 4. attention of the kept rows over the blended cache
  AttnArgs aa{};
  aa.Q = at<void>(ws, L.q);
  aa.qmap = keep_all ? nullptr : at<int>(ws, L.sel);
  aa.qpos = keep_all ? s_in : s_out;
  if (keep_all) {
    aa.fin_ids_in = s_in;
    aa.fin_ids_out = s_out;
    aa.fin_dev_part = sa.dev_part;
    aa.fin_dev = sa.dev;
    aa.fin_n_parts = sa.n_parts;
    aa.fin_ld_part = sa.ld_part;
    aa.fin_n_cand = n_cand;
  }
  aa.K = k_cache;
  aa.V = v_cache;
  aa.O = at<void>(ws, L.o);
  aa.m = m_out;
  aa.T = T;
  aa.n_q = cfg->n_q_heads;
  aa.n_kv = cfg->n_kv_heads;
  aa.hd = D.hd;
  aa.key_split = attn_key_split(dt, m_out, cfg->n_kv_heads, T);
  aa.o_part = at<bf16_t>(ws, L.o_part);
  aa.ml_part = at<float>(ws, L.ml_part);
  st = hip_status(launch_attention(dt, aa, s));
  if (st) return st;
  // 5. O projection, MLP
  return layer_tail(c, w, L, ws, m_out, hidden_in, n_src, keep_all ? nullptr : at<int>(ws, L.sel), in_rows,
                    hidden_out, s, w8, w8 ? &F8 : nullptr);
}

}  // namespace
}  // namespace cb

namespace cb {
namespace {

// Argument checks of a blend call (and validate mode); m_out on success.
cb_status blend_checks(const cb_layer_config* cfg, const cb_layer_weights* w, const cb_rope_dev* rope,
                       void* k_cache, void* v_cache, int32_t T, int32_t n_ctx, int32_t first_chunk_len,
                       const int32_t* s_in, int32_t m_in, const void* hidden_in, const int32_t* in_rows,
                       int32_t k_out, void* hidden_out, int32_t* s_out, void* ws, size_t ws_bytes, void* stream,
                       int* m_out) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  st = check_weights(w);
  if (st) return st;
  if (!k_cache || !v_cache || !s_in || !hidden_in || !hidden_out || !s_out || !ws) return CB_ERR_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(hidden_in) || !aligned16(hidden_out) ||
      !aligned16(ws))
    return CB_ERR_ARG;
  if (T <= 0 || n_ctx < 0 || first_chunk_len < 0 || m_in < 0 || k_out < 0) return CB_ERR_ARG;
  if (n_ctx > T || first_chunk_len > n_ctx) return CB_ERR_SHAPE;
  const int n_query = T - n_ctx;
  const int n_cand = m_in - n_query;
  if (n_cand < 0 || n_cand > n_ctx - first_chunk_len) return CB_ERR_SHAPE;
  if (cfg->dtype == CB_F32 && T > kF32MaxT) return CB_ERR_UNSUPPORTED;
  st = check_rope(cfg, rope, T);
  if (st) return st;
  if (ws_bytes < cb_workspace_size(cfg, T, m_in)) return CB_ERR_WORKSPACE;
  if (t_validate && m_in > 0) {
    st = cb::validate_blend(s_in, m_in, in_rows, T, n_ctx, first_chunk_len, (hipStream_t)stream);
    if (st) return st;
  }
  *m_out = std::min(k_out, n_cand) + n_query;
  return CB_OK;
}

}  // namespace
}  // namespace cb

extern "C" cb_status cb_blend_layer(const cb_layer_config* cfg, const cb_layer_weights* w, const cb_rope_dev* rope,
                                    void* k_cache, void* v_cache, int32_t T, int32_t n_ctx, int32_t first_chunk_len,
                                    const int32_t* s_in, int32_t m_in, const void* hidden_in,
                                    const int32_t* in_rows, int32_t k_out, void* hidden_out, float* dev_out,
                                    int32_t* s_out, int32_t* m_out_host, void* ws, size_t ws_bytes, void* stream) {
  int m_out = 0;
  const cb_status st = cb::blend_checks(cfg, w, rope, k_cache, v_cache, T, n_ctx, first_chunk_len, s_in, m_in,
                                        hidden_in, in_rows, k_out, hidden_out, s_out, ws, ws_bytes, stream, &m_out);
  if (st) return st;
  if (m_out_host) *m_out_host = m_out;
  if (m_in == 0) return CB_OK;
  return cb::blend_run(*cfg, *w, *rope, k_cache, v_cache, T, n_ctx, first_chunk_len, s_in, m_in, hidden_in, in_rows,
                       k_out, hidden_out, dev_out, s_out, ws, (hipStream_t)stream);
}

extern "C" cb_status cb_blend_layer_realign(const cb_layer_config* cfg, const cb_layer_weights* w,
                                            const cb_rope_dev* rope, void* k_cache, void* v_cache, int32_t T,
                                            const int32_t* chunk_offsets, int32_t n_chunks, const int32_t* s_in,
                                            int32_t m_in, const void* hidden_in, const int32_t* in_rows,
                                            int32_t k_out, void* hidden_out, float* dev_out, int32_t* s_out,
                                            int32_t* m_out_host, void* ws, size_t ws_bytes, void* stream) {
  if (!chunk_offsets || n_chunks < 1) return CB_ERR_ARG;
  if (n_chunks > cb::kMaxChunks) return CB_ERR_UNSUPPORTED;
  if (chunk_offsets[0] != 0) return CB_ERR_SHAPE;
  for (int c = 0; c < n_chunks; ++c)
    if (chunk_offsets[c + 1] < chunk_offsets[c]) return CB_ERR_SHAPE;
  if (T < 0 || chunk_offsets[n_chunks] > T) return CB_ERR_SHAPE;
  const int n_ctx = chunk_offsets[n_chunks];
  const int first = n_chunks > 1 ? chunk_offsets[1] : n_ctx;
  int m_out = 0;
  cb_status st = cb::blend_checks(cfg, w, rope, k_cache, v_cache, T, n_ctx, first, s_in, m_in, hidden_in, in_rows,
                                  k_out, hidden_out, s_out, ws, ws_bytes, stream, &m_out);
  if (st) return st;
  if (m_out_host) *m_out_host = m_out;
  const Dims D(*cfg);
  hipStream_t s = (hipStream_t)stream;
  const bool shifts = n_chunks > 1 && n_ctx > first;
  if (m_in == 0) {
    // nothing recomputed: the re-alignment alone
    if (!shifts) return CB_OK;
    return cb_rope_shift(cfg, rope, k_cache, 0, 1, T, chunk_offsets, n_chunks, stream);
  }
  if (!shifts)
    return cb::blend_run(*cfg, *w, *rope, k_cache, v_cache, T, n_ctx, first, s_in, m_in, hidden_in, in_rows, k_out,
                         hidden_out, dev_out, s_out, ws, s);
  cb::ShiftFuse sf{};
  sf.row0 = first;
  sf.row1 = n_ctx;
  sf.n_chunks = n_chunks;
  sf.kv_dim = D.kv_dim;
  sf.hd = D.hd;
  sf.k = k_cache;
  sf.cos = rope->cos;
  sf.sin = rope->sin;
  sf.s_in = s_in;
  sf.m_in = m_in;
  for (int c = 0; c <= n_chunks; ++c) sf.offs.o[c] = chunk_offsets[c];
  return cb::blend_run(*cfg, *w, *rope, k_cache, v_cache, T, n_ctx, first, s_in, m_in, hidden_in, in_rows, k_out,
                       hidden_out, dev_out, s_out, ws, s, nullptr, &sf);
}

extern "C" size_t cb_pack_gateup_size(const cb_layer_config* cfg) {
  if (check_cfg(cfg) != CB_OK || cfg->dtype != CB_BF16) return 0;
  return pack_gateup_bytes(cfg->ffn_dim, cfg->d_model);
}

extern "C" cb_status cb_pack_gateup(const cb_layer_config* cfg, const void* w_gate, const void* w_up, void* packed,
                                    void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != CB_BF16) return CB_ERR_UNSUPPORTED;
  if (!w_gate || !w_up || !packed || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(packed)) return CB_ERR_ARG;
  return hip_status(launch_pack_gateup(w_gate, w_up, cfg->ffn_dim, cfg->d_model, packed, (hipStream_t)stream));
}

extern "C" size_t cb_workspace_size_fp8(const cb_layer_config* cfg, int32_t T, int32_t m_max) {
  if (check_cfg(cfg) != CB_OK || T < 0 || m_max < 0) return 0;
  const int m = std::max(T, m_max);
  return layout_fp8(*cfg, m, align256(layout(*cfg, m, T).total)).total;
}

extern "C" cb_status cb_blend_layer_fp8(const cb_layer_config* cfg, const cb_layer_weights_fp8* w8,
                                        const cb_rope_dev* rope, void* k_cache, void* v_cache, int32_t T,
                                        int32_t n_ctx, int32_t first_chunk_len, const int32_t* s_in, int32_t m_in,
                                        const void* hidden_in, const int32_t* in_rows, int32_t k_out,
                                        void* hidden_out, float* dev_out, int32_t* s_out, int32_t* m_out_host,
                                        void* ws, size_t ws_bytes, void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (!w8) return CB_ERR_ARG;
  {
    const void* p[10] = {w8->attn_norm, w8->w_qkv, w8->e_qkv, w8->w_o,  w8->e_o,
                         w8->mlp_norm,  w8->w_gu,  w8->e_gu,  w8->w_down, w8->e_down};
    for (const void* x : p)
      if (!x) return CB_ERR_ARG;
    if (!aligned16(w8->w_qkv) || !aligned16(w8->w_o) || !aligned16(w8->w_gu) || !aligned16(w8->w_down))
      return CB_ERR_ARG;
  }
  if (cfg->dtype != CB_BF16) return CB_ERR_UNSUPPORTED;
  const Dims D(*cfg);
  if (D.d % 16 || D.q_dim % 16 || D.F % 16) return CB_ERR_SHAPE;
  if (!k_cache || !v_cache || !s_in || !hidden_in || !hidden_out || !s_out || !ws) return CB_ERR_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(hidden_in) || !aligned16(hidden_out) ||
      !aligned16(ws))
    return CB_ERR_ARG;
  if (T <= 0 || n_ctx < 0 || first_chunk_len < 0 || m_in < 0 || k_out < 0) return CB_ERR_ARG;
  if (n_ctx > T || first_chunk_len > n_ctx) return CB_ERR_SHAPE;
  const int n_query = T - n_ctx;
  const int n_cand = m_in - n_query;
  if (n_cand < 0 || n_cand > n_ctx - first_chunk_len) return CB_ERR_SHAPE;
  st = check_rope(cfg, rope, T);
  if (st) return st;
  if (ws_bytes < cb_workspace_size_fp8(cfg, T, m_in)) return CB_ERR_WORKSPACE;
  if (t_validate && m_in > 0) {
    st = cb::validate_blend(s_in, m_in, in_rows, T, n_ctx, first_chunk_len, (hipStream_t)stream);
    if (st) return st;
  }
  const int m_out = std::min(k_out, n_cand) + n_query;
  if (m_out_host) *m_out_host = m_out;
  if (m_in == 0) return CB_OK;
  // the norms as bf16-path weights (the projections come from w8)
  cb_layer_weights wn{};
  wn.attn_norm = w8->attn_norm;
  wn.mlp_norm = w8->mlp_norm;
  return cb::blend_run(*cfg, wn, *rope, k_cache, v_cache, T, n_ctx, first_chunk_len, s_in, m_in, hidden_in, in_rows,
                       k_out, hidden_out, dev_out, s_out, ws, (hipStream_t)stream, w8);
}

extern "C" cb_status cb_full_prefill_layer(const cb_layer_config* cfg, const cb_layer_weights* w,
                                           const cb_rope_dev* rope, const void* hidden_in, int32_t T, int32_t pos0,
                                           void* k_out, void* v_out, void* hidden_out, void* ws, size_t ws_bytes,
                                           void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  st = check_weights(w);
  if (st) return st;
  if (!hidden_in || !k_out || !v_out || !hidden_out || !ws) return CB_ERR_ARG;
  if (!aligned16(hidden_in) || !aligned16(k_out) || !aligned16(v_out) || !aligned16(hidden_out) || !aligned16(ws))
    return CB_ERR_ARG;
  if (T < 0 || pos0 < 0) return CB_ERR_ARG;
  if (cfg->dtype == CB_F32 && T > kF32MaxT) return CB_ERR_UNSUPPORTED;
  st = check_rope(cfg, rope, pos0 + T);
  if (st) return st;
  if (ws_bytes < cb_workspace_size(cfg, T, T)) return CB_ERR_WORKSPACE;
  if (T == 0) return CB_OK;
  const Dims D(*cfg);
  const Ws L = layout(*cfg, T, T);
  hipStream_t s = (hipStream_t)stream;
  const int dt = cfg->dtype;
  GemmArgs g = qkv_args(*cfg, *w, *rope, L, ws, T);
  st = qkv_input(*cfg, *w, g, hidden_in, T, nullptr, T, at<void>(ws, L.xn), true, s);
  if (st) return st;
  g.epi.rows = nullptr;
  g.epi.pos0 = pos0;
  g.epi.k_cache = k_out;
  g.epi.v_cache = v_out;
  g.epi.T = T;
  g.epi.dev_part = nullptr;
  st = hip_status(launch_gemm(dt, g, s));
  if (st) return st;
  AttnArgs aa{};
  aa.Q = at<void>(ws, L.q);
  aa.K = k_out;
  aa.V = v_out;
  aa.O = at<void>(ws, L.o);
  aa.m = T;
  aa.T = T;
  aa.n_q = cfg->n_q_heads;
  aa.n_kv = cfg->n_kv_heads;
  aa.hd = D.hd;
  aa.key_split = attn_key_split(dt, T, cfg->n_kv_heads, T);
  aa.o_part = at<bf16_t>(ws, L.o_part);
  aa.ml_part = at<float>(ws, L.ml_part);
  st = hip_status(launch_attention(dt, aa, s));
  if (st) return st;
  return layer_tail(*cfg, *w, L, ws, T, hidden_in, T, nullptr, nullptr, hidden_out, s);
}

// ---------------------------------------------------------------------------
// the fusor over a stack of layers, with KV loading pipelined with recompute
// ---------------------------------------------------------------------------

namespace {
// staging of one layer's 8-bit K/V (codes, then exponents) on the device
size_t kv8_slot_bytes(const Dims& D, int T) {
  return 2 * align256((size_t)T * D.kv_dim) + 2 * align256((size_t)T * D.n_kv * 4);
}
}  // namespace

extern "C" size_t cb_stack_workspace_size(const cb_layer_config* cfg, int32_t T) {
  if (check_cfg(cfg) != CB_OK || T <= 0) return 0;
  const Dims D(*cfg);
  return align256(cb_workspace_size(cfg, T, T)) + 2 * align256((size_t)T * D.d * D.b) + align256((size_t)T * 4) +
         2 * kv8_slot_bytes(D, T);
}

extern "C" int32_t cb_pick_ratio(double t_prefill_us, double kv_bytes_per_token, int32_t n_tokens,
                                 double link_bytes_per_us, int32_t r_min_e4) {
  if (!(t_prefill_us > 0.0) || !(kv_bytes_per_token > 0.0) || !(link_bytes_per_us > 0.0) || n_tokens <= 0 ||
      r_min_e4 < 0 || r_min_e4 > 10000 || !std::isfinite(t_prefill_us) || !std::isfinite(kv_bytes_per_token) ||
      !std::isfinite(link_bytes_per_us))
    return -1;
  // T_load = bytes per token x tokens / link throughput; T_recompute(r) =
  // r x T_prefill; equal at r_match = T_load / T_prefill
  const double t_load = kv_bytes_per_token * (double)n_tokens / link_bytes_per_us;
  const double r_match = t_load / t_prefill_us;
  const double e4 = std::floor(r_match * 1e4);
  const int32_t r = e4 >= 10000.0 ? 10000 : (int32_t)e4;
  return std::max(r, r_min_e4);
}

namespace {

// where the chunk KV of every layer comes from: nowhere (already in the
// device caches), host copies in the cache dtype, or host 8-bit codes with
// per-(row, KV head) exponents
struct KvSource {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* k_exp = nullptr;
  const int32_t* v_exp = nullptr;
  bool fp8 = false;
};

cb_status stack_run(const cb_layer_config* cfg, int32_t n_layers, const cb_layer_weights* layers,
                    const cb_rope_dev* rope, void* k_caches, void* v_caches, int64_t layer_stride_elems,
                    const KvSource& src, int32_t T, const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift,
                    const void* x_first, const int32_t* ks, int32_t* s_out_all, float* dev_all, void* hidden_out,
                    int32_t* m_rows_host, void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  const void* k_src = src.k;
  const void* v_src = src.v;
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (n_layers < 1 || !layers || !k_caches || !v_caches || !chunk_offsets || !x_first || !ks || !s_out_all ||
      !dev_all || !hidden_out || !ws || T <= 0 || n_chunks < 1)
    return CB_ERR_ARG;
  if ((k_src == nullptr) != (v_src == nullptr)) return CB_ERR_ARG;
  if (src.fp8 && (!k_src || !src.k_exp || !src.v_exp)) return CB_ERR_ARG;
  for (int l = 0; l < n_layers; ++l) {
    st = check_weights(&layers[l]);
    if (st) return st;
    if (ks[l] < 0) return CB_ERR_ARG;
  }
  if (!aligned16(k_caches) || !aligned16(v_caches) || !aligned16(x_first) || !aligned16(hidden_out) ||
      !aligned16(ws))
    return CB_ERR_ARG;
  if (n_chunks > 256) return CB_ERR_UNSUPPORTED;
  if (chunk_offsets[0] != 0) return CB_ERR_SHAPE;
  for (int c = 0; c < n_chunks; ++c)
    if (chunk_offsets[c + 1] < chunk_offsets[c]) return CB_ERR_SHAPE;
  const int n_ctx = chunk_offsets[n_chunks];
  const int L0 = n_chunks > 1 ? chunk_offsets[1] : n_ctx;
  if (n_ctx > T) return CB_ERR_SHAPE;
  if (cfg->dtype == CB_F32 && T > kF32MaxT) return CB_ERR_UNSUPPORTED;
  const Dims D(*cfg);
  const int64_t layer_elems = (int64_t)T * D.kv_dim;
  if (n_layers > 1 && layer_stride_elems < layer_elems) return CB_ERR_SHAPE;
  if ((layer_stride_elems * D.b) % 16) return CB_ERR_ARG;
  if (src.fp8 && D.hd % 16) return CB_ERR_SHAPE;
  st = check_rope(cfg, rope, T);
  if (st) return st;
  if (ws_bytes < cb_stack_workspace_size(cfg, T)) return CB_ERR_WORKSPACE;

  // row counts of every layer, known on the host
  const int n_query = T - n_ctx;
  std::vector<int> m_in(n_layers), m_out(n_layers);
  int rows = T - L0;
  for (int l = 0; l < n_layers; ++l) {
    m_in[l] = rows;
    m_out[l] = std::min(ks[l], rows - n_query) + n_query;
    rows = m_out[l];
  }
  if (m_rows_host)
    for (int l = 0; l < n_layers; ++l) {
      m_rows_host[2 * l] = m_in[l];
      m_rows_host[2 * l + 1] = m_out[l];
    }
  if (m_in[0] == 0) return CB_OK;

  hipStream_t s = (hipStream_t)stream;
  hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : s;
  char* base = (char*)ws;
  const size_t blend_bytes = align256(cb_workspace_size(cfg, T, T));
  const size_t hid_bytes = align256((size_t)T * D.d * D.b);
  void* hid[2] = {base + blend_bytes, base + blend_bytes + hid_bytes};
  int* rows0 = (int*)(base + blend_bytes + 2 * hid_bytes);
  st = hip_status(launch_iota(rows0, m_in[0], L0, s));
  if (st) return st;

  RopeShiftArgs ra{};
  ra.layer_stride = layer_stride_elems;
  ra.T = T;
  ra.kv_dim = D.kv_dim;
  ra.hd = D.hd;
  ra.cos = rope->cos;
  ra.sin = rope->sin;
  ra.offsets = chunk_offsets;
  ra.n_chunks = n_chunks;
  const size_t layer_bytes = (size_t)layer_elems * D.b;
  const int64_t stride_bytes = layer_stride_elems * D.b;

  // KV loading (paper section 5): every layer's copies are queued on the copy
  // stream up front; layer l waits only for its own copies, so the copies of
  // later layers proceed while layer l is recomputed.
  std::vector<hipEvent_t> ev;
  auto cleanup = [&]() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  };
  if (k_src) {
    const bool pipelined = cs != s;
    if (pipelined) {
      // the copies must not start before earlier work on `stream` (which
      // may still read the caches) has finished
      hipEvent_t e0 = nullptr;
      if ((st = hip_status(hipEventCreateWithFlags(&e0, hipEventDisableTiming)))) return st;
      ev.push_back(e0);
      if ((st = hip_status(hipEventRecord(e0, s))) || (st = hip_status(hipStreamWaitEvent(cs, e0, 0)))) {
        cleanup();
        return st;
      }
    }
    // 8-bit sources: two staging slots after the hidden-row buffers; layer
    // l's codes go to slot l % 2 and are expanded (keys re-aligned) into its
    // caches on the copy stream, which also orders the slot's reuse
    char* stage0 = base + blend_bytes + 2 * hid_bytes + align256((size_t)T * 4);
    const size_t code_bytes = (size_t)T * D.kv_dim, exp_bytes = (size_t)T * D.n_kv * 4;
    for (int l = 0; l < n_layers; ++l) {
      char* kd = (char*)k_caches + (int64_t)l * stride_bytes;
      char* vd = (char*)v_caches + (int64_t)l * stride_bytes;
      if (src.fp8) {
        char* slot = stage0 + (l & 1) * kv8_slot_bytes(D, T);
        uint8_t* kc8 = (uint8_t*)slot;
        uint8_t* vc8 = (uint8_t*)(slot + align256(code_bytes));
        int32_t* ke = (int32_t*)(slot + 2 * align256(code_bytes));
        int32_t* ve = (int32_t*)(slot + 2 * align256(code_bytes) + align256(exp_bytes));
        const char* kh = (const char*)k_src + (int64_t)l * code_bytes;
        const char* vh = (const char*)v_src + (int64_t)l * code_bytes;
        const int32_t* keh = src.k_exp + (int64_t)l * T * D.n_kv;
        const int32_t* veh = src.v_exp + (int64_t)l * T * D.n_kv;
        if ((st = hip_status(hipMemcpyAsync(kc8, kh, code_bytes, hipMemcpyHostToDevice, cs))) ||
            (st = hip_status(hipMemcpyAsync(vc8, vh, code_bytes, hipMemcpyHostToDevice, cs))) ||
            (st = hip_status(hipMemcpyAsync(ke, keh, exp_bytes, hipMemcpyHostToDevice, cs))) ||
            (st = hip_status(hipMemcpyAsync(ve, veh, exp_bytes, hipMemcpyHostToDevice, cs)))) {
          cleanup();
          return st;
        }
        KvExpandArgs xa{};
        xa.k_codes = kc8;
        xa.v_codes = vc8;
        xa.k_exps = ke;
        xa.v_exps = ve;
        xa.k_cache = kd;
        xa.v_cache = vd;
        xa.layer_stride = layer_stride_elems;
        xa.n_layers = 1;
        xa.row0 = 0;
        xa.n_rows = T;
        xa.kv_dim = D.kv_dim;
        xa.n_kv = D.n_kv;
        xa.hd = D.hd;
        xa.cos = rope->cos;
        xa.sin = rope->sin;
        xa.n_chunks = n_chunks;
        xa.shift = shift;
        if ((st = hip_status(launch_kv_expand(cfg->dtype, xa, chunk_offsets, cs)))) {
          cleanup();
          return st;
        }
      } else {
        const char* kh = (const char*)k_src + (int64_t)l * layer_bytes;
        const char* vh = (const char*)v_src + (int64_t)l * layer_bytes;
        if ((st = hip_status(hipMemcpyAsync(kd, kh, layer_bytes, hipMemcpyHostToDevice, cs))) ||
            (st = hip_status(hipMemcpyAsync(vd, vh, layer_bytes, hipMemcpyHostToDevice, cs)))) {
          cleanup();
          return st;
        }
      }
      if (pipelined) {
        hipEvent_t e = nullptr;
        if ((st = hip_status(hipEventCreateWithFlags(&e, hipEventDisableTiming)))) {
          cleanup();
          return st;
        }
        ev.push_back(e);
        if ((st = hip_status(hipEventRecord(e, cs)))) {
          cleanup();
          return st;
        }
      }
    }
  } else if (shift) {
    // caches already on the device: one re-alignment launch for all layers
    ra.k_cache = k_caches;
    ra.n_layers = n_layers;
    if ((st = hip_status(launch_rope_shift(cfg->dtype, ra, s)))) return st;
  }

  int64_t off_in = 0, off_out = 0;
  for (int l = 0; l < n_layers; ++l) {
    void* kc = (char*)k_caches + (int64_t)l * stride_bytes;
    void* vc = (char*)v_caches + (int64_t)l * stride_bytes;
    if (k_src) {
      if (ev.size() > 1 && (st = hip_status(hipStreamWaitEvent(s, ev[1 + l], 0)))) {
        cleanup();
        return st;
      }
      if (shift && !src.fp8) {
        ra.k_cache = kc;
        ra.n_layers = 1;
        if ((st = hip_status(launch_rope_shift(cfg->dtype, ra, s)))) {
          cleanup();
          return st;
        }
      }
    }
    if (m_in[l] == 0) continue;   // nothing left to recompute (no query rows, k = 0)
    const int32_t* s_in = l == 0 ? rows0 : s_out_all + (off_out - m_out[l - 1]);
    const void* x = l == 0 ? x_first : hid[(l - 1) & 1];
    void* y = l == n_layers - 1 ? hidden_out : hid[l & 1];
    st = blend_run(*cfg, layers[l], *rope, kc, vc, T, n_ctx, L0, s_in, m_in[l], x, nullptr, ks[l], y,
                   dev_all + off_in, s_out_all + off_out, base, s);
    if (st) {
      cleanup();
      return st;
    }
    off_in += m_in[l];
    off_out += m_out[l];
  }
  cleanup();
  return CB_OK;
}

}  // namespace

extern "C" cb_status cb_blend_stack(const cb_layer_config* cfg, int32_t n_layers, const cb_layer_weights* layers,
                                    const cb_rope_dev* rope, void* k_caches, void* v_caches,
                                    int64_t layer_stride_elems, const void* k_src, const void* v_src, int32_t T,
                                    const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift,
                                    const void* x_first, const int32_t* ks, int32_t* s_out_all, float* dev_all,
                                    void* hidden_out, int32_t* m_rows_host, void* ws, size_t ws_bytes, void* stream,
                                    void* copy_stream) {
  KvSource src;
  src.k = k_src;
  src.v = v_src;
  return stack_run(cfg, n_layers, layers, rope, k_caches, v_caches, layer_stride_elems, src, T, chunk_offsets,
                   n_chunks, shift, x_first, ks, s_out_all, dev_all, hidden_out, m_rows_host, ws, ws_bytes, stream,
                   copy_stream);
}

extern "C" cb_status cb_blend_stack_kv8(const cb_layer_config* cfg, int32_t n_layers, const cb_layer_weights* layers,
                                        const cb_rope_dev* rope, void* k_caches, void* v_caches,
                                        int64_t layer_stride_elems, const uint8_t* k_src, const int32_t* k_src_exp,
                                        const uint8_t* v_src, const int32_t* v_src_exp, int32_t T,
                                        const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift,
                                        const void* x_first, const int32_t* ks, int32_t* s_out_all, float* dev_all,
                                        void* hidden_out, int32_t* m_rows_host, void* ws, size_t ws_bytes,
                                        void* stream, void* copy_stream) {
  if (!k_src || !v_src || !k_src_exp || !v_src_exp) return CB_ERR_ARG;
  KvSource src;
  src.k = k_src;
  src.v = v_src;
  src.k_exp = k_src_exp;
  src.v_exp = v_src_exp;
  src.fp8 = true;
  return stack_run(cfg, n_layers, layers, rope, k_caches, v_caches, layer_stride_elems, src, T, chunk_offsets,
                   n_chunks, shift, x_first, ks, s_out_all, dev_all, hidden_out, m_rows_host, ws, ws_bytes, stream,
                   copy_stream);
}

extern "C" cb_status cb_kv_from_fp8(const cb_layer_config* cfg, const cb_rope_dev* rope, const uint8_t* k_codes,
                                    const int32_t* k_exps, const uint8_t* v_codes, const int32_t* v_exps,
                                    int32_t n_layers, int32_t row_begin, int32_t n_rows, void* k_cache,
                                    void* v_cache, int64_t layer_stride_elems, int32_t T,
                                    const int32_t* chunk_offsets, int32_t n_chunks, int32_t shift, void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (!k_codes || !k_exps || !v_codes || !v_exps || !k_cache || !v_cache || !chunk_offsets || n_layers < 0 ||
      row_begin < 0 || n_rows < 0 || T < 0 || n_chunks < 1)
    return CB_ERR_ARG;
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_cache) || !aligned16(v_cache)) return CB_ERR_ARG;
  if (n_chunks > kMaxShiftChunks) return CB_ERR_UNSUPPORTED;
  if (chunk_offsets[0] != 0) return CB_ERR_SHAPE;
  for (int c = 0; c < n_chunks; ++c)
    if (chunk_offsets[c + 1] < chunk_offsets[c]) return CB_ERR_SHAPE;
  if (chunk_offsets[n_chunks] > T || (int64_t)row_begin + n_rows > T) return CB_ERR_SHAPE;
  const Dims D(*cfg);
  if (D.hd % 16) return CB_ERR_SHAPE;
  if (n_layers > 1 && layer_stride_elems < (int64_t)T * D.kv_dim) return CB_ERR_SHAPE;
  if ((layer_stride_elems * D.b) % 16) return CB_ERR_ARG;
  if (shift) {
    st = check_rope(cfg, rope, n_chunks > 1 ? chunk_offsets[n_chunks - 1] + 1 : 0);
    if (st) return st;
  }
  KvExpandArgs a{};
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_exps = k_exps;
  a.v_exps = v_exps;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.layer_stride = layer_stride_elems;
  a.n_layers = n_layers;
  a.row0 = row_begin;
  a.n_rows = n_rows;
  a.kv_dim = D.kv_dim;
  a.n_kv = D.n_kv;
  a.hd = D.hd;
  a.cos = shift ? rope->cos : nullptr;
  a.sin = shift ? rope->sin : nullptr;
  a.n_chunks = n_chunks;
  a.shift = shift;
  return hip_status(launch_kv_expand(cfg->dtype, a, chunk_offsets, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// several requests in one fusor layer
// ---------------------------------------------------------------------------

extern "C" cb_status cb_blend_batch(const cb_layer_config* cfg, const cb_layer_weights* w, const cb_rope_dev* rope,
                                    int32_t n_req, const cb_blend_request* reqs, const int32_t* s_in,
                                    const void* hidden_in, void* hidden_out, float* dev_out, int32_t* s_out,
                                    int32_t* m_out_host, void* ws, size_t ws_bytes, void* stream) {
  cb_status st = check_cfg(cfg);
  if (st) return st;
  st = check_weights(w);
  if (st) return st;
  if (n_req < 1 || !reqs || !s_in || !hidden_in || !hidden_out || !s_out || !ws) return CB_ERR_ARG;
  if (n_req > kMaxReq) return CB_ERR_UNSUPPORTED;
  if (!aligned16(hidden_in) || !aligned16(hidden_out) || !aligned16(ws)) return CB_ERR_ARG;
  int T_max = 1, M_in = 0, M_out = 0, tiles = 0;
  std::vector<int> n_cand(n_req), m_out(n_req);
  for (int r = 0; r < n_req; ++r) {
    const cb_blend_request& q = reqs[r];
    if (!q.k_cache || !q.v_cache || !aligned16(q.k_cache) || !aligned16(q.v_cache)) return CB_ERR_ARG;
    if (q.T <= 0 || q.n_ctx < 0 || q.first_chunk_len < 0 || q.m_in < 0 || q.k_out < 0) return CB_ERR_ARG;
    if (q.n_ctx > q.T || q.first_chunk_len > q.n_ctx) return CB_ERR_SHAPE;
    n_cand[r] = q.m_in - (q.T - q.n_ctx);
    if (n_cand[r] < 0 || n_cand[r] > q.n_ctx - q.first_chunk_len) return CB_ERR_SHAPE;
    if (cfg->dtype == CB_F32 && q.T > kF32MaxT) return CB_ERR_UNSUPPORTED;
    m_out[r] = std::min(q.k_out, n_cand[r]) + (q.T - q.n_ctx);
    T_max = std::max(T_max, (int)q.T);
    M_in += q.m_in;
    M_out += m_out[r];
    tiles += (m_out[r] + kAttnRowTile - 1) / kAttnRowTile;
  }
  st = check_rope(cfg, rope, T_max);
  if (st) return st;
  if (ws_bytes < cb_workspace_size(cfg, T_max, M_in)) return CB_ERR_WORKSPACE;
  if (t_validate && M_in > 0) {
    std::vector<int32_t> rows;
    if (!cb::fetch(rows, s_in, M_in, (hipStream_t)stream)) return CB_ERR_HIP;
    int off = 0;
    for (int r = 0; r < n_req; ++r) {
      const cb_blend_request& q = reqs[r];
      st = cb::check_rows(rows.data() + off, q.m_in, q.T, q.n_ctx, q.first_chunk_len);
      if (st) return st;
      off += q.m_in;
    }
  }
  if (m_out_host)
    for (int r = 0; r < n_req; ++r) m_out_host[r] = m_out[r];
  if (M_in == 0) return CB_OK;

  const cb_layer_config& c = *cfg;
  const Dims D(c);
  const Ws L = layout(c, std::max(T_max, M_in), T_max);
  hipStream_t s = (hipStream_t)stream;
  const int dt = c.dtype;
  // 1-2. attention RMSNorm of every request's rows, one QKV GEMM over all
  // rows; each row's epilogue uses its own request's cache
  GemmArgs g = qkv_args(c, *w, *rope, L, ws, M_in);
  st = qkv_input(c, *w, g, hidden_in, M_in, nullptr, M_in, at<void>(ws, L.xn), true, s);
  if (st) return st;
  g.epi.rows = s_in;
  g.epi.pos0 = 0;
  g.epi.k_cache = reqs[0].k_cache;
  g.epi.v_cache = reqs[0].v_cache;
  g.epi.T = T_max;
  g.epi.dev_part = at<float>(ws, L.devp);
  ReqTable& rq = g.epi.req;
  rq.n = n_req;
  int off = 0;
  for (int r = 0; r < n_req; ++r) {
    rq.row_off[r] = off;
    rq.k[r] = reqs[r].k_cache;
    rq.v[r] = reqs[r].v_cache;
    rq.T[r] = reqs[r].T;
    rq.lo[r] = reqs[r].first_chunk_len;
    rq.hi[r] = reqs[r].n_ctx;
    off += reqs[r].m_in;
  }
  rq.row_off[n_req] = off;
  st = hip_status(launch_gemm(dt, g, s));
  if (st) return st;
  // 3. one top-k per request
  SelectArgs sa{};
  sa.dev_part = at<float>(ws, L.devp);
  sa.n_parts = D.n_k_tiles();
  sa.ld_part = M_in;
  sa.dev = dev_out ? dev_out : at<float>(ws, L.dev);
  sa.n_cand = n_cand[0];
  sa.m_in = reqs[0].m_in;
  sa.k = reqs[0].k_out;
  sa.ids_in = s_in;
  sa.sel = at<int>(ws, L.sel);
  sa.ids_out = s_out;
  sa.n_seg = n_req;
  int in_off = 0, out_off = 0;
  for (int r = 0; r < n_req; ++r) {
    sa.seg[r] = SelectArgs::Seg{in_off, reqs[r].m_in, n_cand[r], reqs[r].k_out, out_off};
    in_off += reqs[r].m_in;
    out_off += m_out[r];
  }
  st = hip_status(launch_select(sa, s));
  if (st) return st;
  // 4. attention: row tiles never straddle two requests
  AttnArgs aa{};
  aa.Q = at<void>(ws, L.q);
  aa.qmap = at<int>(ws, L.sel);
  aa.qpos = s_out;
  aa.K = reqs[0].k_cache;
  aa.V = reqs[0].v_cache;
  aa.O = at<void>(ws, L.o);
  aa.m = M_out;
  aa.T = T_max;
  aa.n_q = c.n_q_heads;
  aa.n_kv = c.n_kv_heads;
  aa.hd = D.hd;
  aa.key_split = attn_key_split(dt, tiles * kAttnRowTile, c.n_kv_heads, T_max);
  aa.o_part = at<bf16_t>(ws, L.o_part);
  aa.ml_part = at<float>(ws, L.ml_part);
  aa.req.n = n_req;
  int ro = 0, to = 0;
  for (int r = 0; r < n_req; ++r) {
    aa.req.row_off[r] = ro;
    aa.req.tile_off[r] = to;
    aa.req.k[r] = reqs[r].k_cache;
    aa.req.v[r] = reqs[r].v_cache;
    aa.req.T[r] = reqs[r].T;
    ro += m_out[r];
    to += (m_out[r] + kAttnRowTile - 1) / kAttnRowTile;
  }
  aa.req.row_off[n_req] = ro;
  aa.req.tile_off[n_req] = to;
  if (M_out > 0) {
    st = hip_status(launch_attention(dt, aa, s));
    if (st) return st;
  }
  // 5. O projection, MLP over all kept rows (residual rows via the selection)
  return layer_tail(c, *w, L, ws, M_out, hidden_in, M_in, at<int>(ws, L.sel), nullptr, hidden_out, s);
}

// ---------------------------------------------------------------------------
// fp8 E4M3 operands
// ---------------------------------------------------------------------------

extern "C" cb_status cb_quantize_fp8(int32_t src_dtype, const void* x, int32_t rows, int32_t cols, uint8_t* codes,
                                     int32_t* exps, void* stream) {
  if (src_dtype != CB_F32 && src_dtype != CB_BF16) return CB_ERR_ARG;
  if (rows < 0 || cols < 0 || (rows > 0 && (!x || !codes || !exps))) return CB_ERR_ARG;
  if (rows == 0 || cols == 0) return CB_OK;
  return hip_status(launch_quantize_rows(src_dtype, x, rows, cols, codes, exps, (hipStream_t)stream));
}

extern "C" size_t cb_gemm_fp8_workspace_size(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  const int s = fp8_splits(N, K);
  return s > 1 ? (size_t)s * M * N * 4 : 0;
}

extern "C" cb_status cb_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* a, const int32_t* a_exp,
                                 const uint8_t* b, const int32_t* b_exp, void* c, int32_t ldc, int32_t out_dtype,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0 || ldc < N) return CB_ERR_ARG;
  if (out_dtype != CB_F32 && out_dtype != CB_BF16) return CB_ERR_ARG;
  if (M == 0 || N == 0) return CB_OK;
  if (!a || !a_exp || !b || !b_exp || !c) return CB_ERR_ARG;
  if (K % 16 || !aligned16(a) || !aligned16(b)) return CB_ERR_SHAPE;
  if ((int64_t)M * K >= (int64_t)1 << 31 || (int64_t)N * K >= (int64_t)1 << 31) return CB_ERR_UNSUPPORTED;
  Fp8GemmArgs g{};
  g.A = a;
  g.a_exp = a_exp;
  g.B = b;
  g.b_exp = b_exp;
  g.C = c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.splits = fp8_splits(N, K);
  if (g.splits > 1) {
    if (!ws || ws_bytes < cb_gemm_fp8_workspace_size(M, N, K)) return CB_ERR_WORKSPACE;
    g.part = (float*)ws;
  }
  return hip_status(launch_gemm_fp8(g, out_dtype, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// cb_gemm_fp8_noalloc: the split-K partials in a static device array
// ---------------------------------------------------------------------------
namespace cb {
namespace {

constexpr int kMaxScratchDevices = 64;

// One copy per GPU, alive until the process ends.  Host code never uses this
// name as an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[CB_GEMM_FP8_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch`.
cb_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return CB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return CB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CB_OK;
}

}  // namespace
}  // namespace cb

extern "C" cb_status cb_gemm_fp8_noalloc(int32_t M, int32_t N, int32_t K, const uint8_t* a, const int32_t* a_exp,
                                         const uint8_t* b, const int32_t* b_exp, void* c, int32_t ldc,
                                         int32_t out_dtype, void* stream) {
  using namespace cb;
  // the same checks as cb_gemm_fp8, then the scratch limit, all before any HIP call
  if (M < 0 || N < 0 || K < 0 || ldc < N) return CB_ERR_ARG;
  if (out_dtype != CB_F32 && out_dtype != CB_BF16) return CB_ERR_ARG;
  if (M == 0 || N == 0) return CB_OK;
  if (!a || !a_exp || !b || !b_exp || !c) return CB_ERR_ARG;
  if (K % 16 || !aligned16(a) || !aligned16(b)) return CB_ERR_SHAPE;
  if ((int64_t)M * K >= (int64_t)1 << 31 || (int64_t)N * K >= (int64_t)1 << 31) return CB_ERR_UNSUPPORTED;
  const size_t need = cb_gemm_fp8_workspace_size(M, N, K);
  if (need > (size_t)CB_GEMM_FP8_SCRATCH_BYTES) return CB_ERR_WORKSPACE;
  Fp8GemmArgs g{};
  g.A = a;
  g.a_exp = a_exp;
  g.B = b;
  g.b_exp = b_exp;
  g.C = c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.splits = fp8_splits(N, K);
  if (g.splits > 1) {
    // every partial the finishing pass reads is written first by the same
    // launch sequence, so nothing has to start at zero
    void* p = nullptr;
    const cb_status st = static_scratch(&p);
    if (st) return st;
    g.part = (float*)p;
  }
  return hip_status(launch_gemm_fp8(g, out_dtype, (hipStream_t)stream));
}

extern "C" cb_status cb_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  using namespace cb;
  if (bytes == 0) return CB_OK;
  if (!src || !dst || bytes % 16 || !aligned16(src) || !aligned16(dst)) return CB_ERR_ARG;
  return hip_status(launch_stream_copy(src, dst, bytes, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// deviation analytics
// ---------------------------------------------------------------------------

extern "C" size_t cb_workspace_q_offset(const cb_layer_config* cfg, int32_t T) {
  using namespace cb;
  if (check_cfg(cfg) != CB_OK || T <= 0) return 0;
  return layout(*cfg, T, T).q;
}

extern "C" size_t cb_analytics_workspace_size(int32_t m, int32_t n_q, int32_t n) {
  if (m < 0 || n_q < 0 || n < 0) return 0;
  const size_t a = (size_t)m * n_q * 2, b = (size_t)n * 2;
  return (a > b ? a : b) * sizeof(double) + 256;
}

extern "C" cb_status cb_attention_deviation(const cb_layer_config* cfg, int32_t m, const void* q_a, const void* k_a,
                                            const void* q_b, const void* k_b, int32_t T, const int32_t* last_key,
                                            double* out, void* ws, size_t ws_bytes, void* stream) {
  using namespace cb;
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (m < 0 || T <= 0 || !out) return CB_ERR_ARG;
  if (m == 0) return CB_OK;
  if (!q_a || !k_a || !q_b || !k_b || !last_key || !ws) return CB_ERR_ARG;
  if (ws_bytes < cb_analytics_workspace_size(m, cfg->n_q_heads, 0)) return CB_ERR_WORKSPACE;
  return hip_status(launch_attention_deviation(cfg->dtype, m, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, q_a,
                                               k_a, q_b, k_b, T, last_key, (double*)ws, out, (hipStream_t)stream));
}

extern "C" cb_status cb_spearman(const float* x, const float* y, int32_t n, double* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  using namespace cb;
  if (n <= 0 || !x || !y || !out || !ws) return CB_ERR_ARG;
  if (ws_bytes < cb_analytics_workspace_size(0, 0, n)) return CB_ERR_WORKSPACE;
  return hip_status(launch_spearman(x, y, n, (double*)ws, out, (hipStream_t)stream));
}

extern "C" cb_status cb_top_share(const float* x, int32_t n, int32_t k, double* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  using namespace cb;
  if (n <= 0 || k < 0 || k > n || !x || !out || !ws) return CB_ERR_ARG;
  if (ws_bytes < cb_analytics_workspace_size(0, 0, n)) return CB_ERR_WORKSPACE;
  return hip_status(launch_top_share(x, n, k, (double*)ws, out, (hipStream_t)stream));
}

extern "C" size_t cb_fold_qkv_size(const cb_layer_config* cfg) {
  using namespace cb;
  if (check_cfg(cfg) != CB_OK || cfg->dtype != CB_BF16) return 0;
  const Dims D(*cfg);
  return (size_t)D.n_qkv() * D.d * 2;
}

extern "C" cb_status cb_fold_qkv(const cb_layer_config* cfg, const cb_layer_weights* w, void* out, void* stream) {
  using namespace cb;
  cb_status st = check_cfg(cfg);
  if (st) return st;
  if (cfg->dtype != CB_BF16) return CB_ERR_UNSUPPORTED;
  if (!w || !w->w_q || !w->w_k || !w->w_v || !w->attn_norm || !out || !aligned16(out) || !aligned16(w->w_q) ||
      !aligned16(w->w_k) || !aligned16(w->w_v) || !aligned16(w->attn_norm))
    return CB_ERR_ARG;
  const Dims D(*cfg);
  return hip_status(launch_fold_qkv(w->w_q, w->w_k, w->w_v, D.q_dim, D.kv_dim, D.d, (const float*)w->attn_norm, out,
                                    (hipStream_t)stream));
}
