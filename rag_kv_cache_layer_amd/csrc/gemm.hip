// Projections of the recomputed rows: C[M][N] = A[M][K] * B[N][K]^T.
//
// CacheBlend (arXiv 2405.16444) section 4.2, Figure 5b: only the selected
// tokens' rows go through the layer's projections, so these are dense
// contractions with a small M (the selected rows) against the full weight
// matrices -- the part of the fusor that really is GEMM-shaped.  B is the
// nn.Linear weight [out][in], so both operands are contiguous along K.
//
// bf16 path (gfx950 matrix cores).  Operand tiles go from HBM/L2 straight to
// LDS with buffer loads that write LDS (no VGPR staging); a buffer resource
// per operand turns rows past the matrix and K past the split into zero
// fills.  Rows of the LDS tiles are XOR-swizzled by 16-byte chunk so the
// 16-row fragment reads hit every bank once.  A ring of LDS stages keeps
// several K steps in flight; each wave waits only for its own loads of the
// step it needs (vmcnt) and then meets the others at a plain barrier (a fenced
// barrier would drain the ring).  Two tile shapes:
//  * 128x128, K step 64, 4-stage ring, four waves of 64x64 (4x4 blocks of
//    v_mfma_f32_16x16x32_bf16): QKV, O and down projections;
//  * 256x256, K step 32, 4-stage ring, eight waves of 128x64 (four waves of
//    128x128 with the accumulators in AGPRs as a build option): the gate/up
//    projection, where N is large -- four times the matrix work per barrier.
// Tiles are numbered so that the M tiles sharing one weight tile run back to
// back on the same XCD (workgroups are dealt round-robin to the 8 XCDs),
// which keeps each weight tile in that XCD's L2 while it is reused.  Split-K
// (chosen from N and K only, never from M) writes fp32 partials that a
// second, LDS-free kernel adds in split order before the epilogue, so a
// row's result never depends on how many rows there are.
//
// fp32 path: a 64x64 SIMT tile kernel (exact fp32 products, fp32 accumulate)
// for the fp32 configuration.
//
// Epilogues (applied from an fp32 tile in LDS, 8 consecutive columns per
// thread): QKV (RoPE at each row's absolute position on Q and K, per-row K
// deviation against the cached row before it is replaced, scatter of K/V into
// the cache), residual add, and SwiGLU on interleaved gate/up tiles.
#include <algorithm>
#include <type_traits>

#include "cb_internal.h"

namespace cb {

namespace {

// bf16 tiles
constexpr int BM = 128, BN = 128, BK = 64, CLD = BN + 4;
// fp32 tiles
constexpr int FBM = 64, FBN = 64, FBK = 16, FCLD = FBN + 4;

// Pointer to row j of output tile tn of the (virtual) B matrix; NULL when the
// row is past the end.
template <typename T>
__device__ __forceinline__ const T* b_row(const BOperand& B, int K, int N, int tn, int bn, int j) {
  if (B.mode == 0) {
    const int c = tn * bn + j;
    if (c >= N) return nullptr;
    if (c < B.n1) return (const T*)B.p0 + (int64_t)c * K;
    if (c < B.n2) return (const T*)B.p1 + (int64_t)(c - B.n1) * K;
    return (const T*)B.p2 + (int64_t)(c - B.n2) * K;
  }
  const int half = bn / 2;
  const int f = tn * half + (j % half);
  if (f >= B.n_feat) return nullptr;
  return (const T*)(j < half ? B.p0 : B.p1) + (int64_t)f * K;
}

// ---------------------------------------------------------------------------
// epilogues
// ---------------------------------------------------------------------------

__device__ __forceinline__ void rope8(float v[8], const float* cs, const float* sn) {
  // two rounded products and one rounded sum per output, in every epilogue
  // that applies it
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = v[2 * j], b = v[2 * j + 1];
    v[2 * j] = a * cs[j] - b * sn[j];
    v[2 * j + 1] = a * sn[j] + b * cs[j];
  }
}

// Sum of squared differences of 8 new and cached key values, added to acc in
// element order with one fused multiply-add each (the same in every
// epilogue that takes the deviation).
__device__ __forceinline__ float dev_add8(const float r[8], const float old[8], float acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = r[j] - old[j];
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc;
}

// Q/K/V columns: returns this group's contribution to the row's K deviation.
// With sf (re-alignment in the same launch) the cached key still sits at its
// chunk-local position: it is rotated by its chunk's offset and rounded to
// the cache type, exactly as the shift stores it, before the comparison.
template <typename T>
__device__ float epi_qkv(const EpiParams& e, int gm, int c, float v[8], const ShiftFuse* sf) {
  const int crow = e.rows ? e.rows[gm] : gm;
  void* k_cache = e.k_cache;
  void* v_cache = e.v_cache;
  int n_rows = e.T, dev_lo = e.dev_lo, dev_hi = e.dev_hi;
  if (e.req.n > 0) {
    const int r = req_of_row(e.req, gm);
    k_cache = e.req.k[r];
    v_cache = e.req.v[r];
    n_rows = e.req.T[r];
    dev_lo = e.req.lo[r];
    dev_hi = e.req.hi[r];
  }
  if (crow < 0 || crow >= n_rows) return 0.f;
  const int pos = crow + e.pos0;
  if (c < e.q_dim + e.kv_dim) {
    const int dim = (c < e.q_dim ? c : c - e.q_dim) % e.hd;
    const int64_t t = (int64_t)pos * (e.hd / 2) + dim / 2;
    rope8(v, e.cos + t, e.sin + t);
  }
  if (c < e.q_dim) {
    store8((T*)e.q_out + (int64_t)gm * e.q_dim + c, v);
    return 0.f;
  }
  if (c < e.q_dim + e.kv_dim) {
    T* kp = (T*)k_cache + (int64_t)crow * e.kv_dim + (c - e.q_dim);
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = Elem<T>::rnd(v[j]);
    float contrib = 0.f;
    if (e.dev_part && crow >= dev_lo && crow < dev_hi) {
      float old[8];
      load8(kp, old);
      if (sf) {
        const int delta = chunk_delta_scan(sf->offs, sf->n_chunks, crow);
        const int64_t t = (int64_t)delta * (e.hd / 2) + ((c - e.q_dim) % e.hd) / 2;
        float rot[8];
        rope_rotate8(old, sf->cos + t, sf->sin + t, rot);
#pragma unroll
        for (int j = 0; j < 8; ++j) old[j] = Elem<T>::rnd(rot[j]);
      }
      contrib = dev_add8(r, old, contrib);
    }
    store8(kp, r);
    return contrib;
  }
  store8((T*)v_cache + (int64_t)crow * e.kv_dim + (c - e.q_dim - e.kv_dim), v);
  return 0.f;
}

template <typename T>
__device__ void epi_resid(const EpiParams& e, int gm, int c, const float v[8]) {
  const int r = map_row(gm, e.rmap1, e.rmap2);
  float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r >= 0 && r < e.T) {
    if (e.resid_f32) load8((const float*)e.resid + (int64_t)r * e.ld_out + c, x);
    else load8((const T*)e.resid + (int64_t)r * e.ld_out + c, x);
  }
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = x[j] + v[j];
  if (e.out_f32) store8((float*)e.out + (int64_t)gm * e.ld_out + c, o);
  else store8((T*)e.out + (int64_t)gm * e.ld_out + c, o);
}

template <typename T>
__device__ void epi_swiglu(const EpiParams& e, int gm, int f, const float g[8], const float u[8]) {
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = silu(g[j]) * u[j];
  store8((T*)e.out + (int64_t)gm * e.ld_out + f, o);
}

template <typename T>
__device__ void epi_store(const EpiParams& e, int gm, int c, const float v[8]) {
  if (e.out_f32) store8((float*)e.out + (int64_t)gm * e.ld_out + c, v);
  else store8((T*)e.out + (int64_t)gm * e.ld_out + c, v);
}

// The QKV epilogue of a whole bm x bn tile for a single-request call, in
// three phases so that a thread's memory reads for all of its rows are in
// flight together: the rows' cache indices; then the RoPE table entries and
// (deviation columns) the cached keys; then, row by row, the arithmetic and
// the stores -- per element the same operations in the same order as
// epi_qkv, so the results are identical.  RoPE tables are 16-byte aligned
// (checked at the boundary), so a thread's four cos / sin entries are one
// 16-byte load each.
template <typename T, int bm, int bn, int NT>
__device__ void qkv_tile_epilogue(const EpiParams& e, const float* Cs, int cld, int m0, int tn, int M, int N,
                                  const float* row_scale, const ShiftFuse* sf) {
  constexpr int tpr = bn / 8;           // threads per row (16 for 128 columns)
  constexpr int rpp = NT / tpr;         // rows per pass
  constexpr int NP = bm / rpp;          // passes
  static_assert(NT % tpr == 0 && bm % rpp == 0, "whole passes");
  const int tid = threadIdx.x;
  const int lr = tid / tpr, lc = (tid % tpr) * 8;
  const int c = tn * bn + lc;
  const bool col_ok = c < N;
  const bool is_q = c < e.q_dim;
  const bool is_k = !is_q && c < e.q_dim + e.kv_dim;
  const bool rope_col = c < e.q_dim + e.kv_dim;
  const int dim = (is_q ? c : c - e.q_dim) % e.hd;
  const bool k_tile = e.dev_part != nullptr && tn * bn < e.q_dim + e.kv_dim && tn * bn + bn > e.q_dim;
  int crow[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int gm = m0 + p * rpp + lr;
    int r = -1;
    if (gm < M && col_ok) r = e.rows ? e.rows[gm] : gm;
    crow[p] = (r >= 0 && r < e.T) ? r : -1;
  }
  float4 cs[NP], sn[NP], cd[NP], sd[NP];
  uint4 oldk[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = crow[p];
    if (r >= 0 && rope_col) {
      const int64_t t = (int64_t)(r + e.pos0) * (e.hd / 2) + dim / 2;
      cs[p] = *reinterpret_cast<const float4*>(e.cos + t);
      sn[p] = *reinterpret_cast<const float4*>(e.sin + t);
    }
    if (r >= 0 && is_k && e.dev_part && r >= e.dev_lo && r < e.dev_hi) {
      oldk[p] = *reinterpret_cast<const uint4*>((const T*)e.k_cache + (int64_t)r * e.kv_dim + (c - e.q_dim));
      if (sf) {
        const int delta = chunk_delta_scan(sf->offs, sf->n_chunks, r);
        const int64_t t = (int64_t)delta * (e.hd / 2) + dim / 2;
        cd[p] = *reinterpret_cast<const float4*>(sf->cos + t);
        sd[p] = *reinterpret_cast<const float4*>(sf->sin + t);
      }
    }
  }
  float contrib[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int rl = p * rpp + lr;
    const int gm = m0 + rl;
    const int r = crow[p];
    contrib[p] = 0.f;
    if (r >= 0) {
      const float* row = Cs + rl * cld;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = row[lc + j];
      if (row_scale) {
        const float rs = row_scale[rl];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= rs;
      }
      if (rope_col) {
        const float ca[4] = {cs[p].x, cs[p].y, cs[p].z, cs[p].w};
        const float sa[4] = {sn[p].x, sn[p].y, sn[p].z, sn[p].w};
        rope8(v, ca, sa);
      }
      if (is_q) {
        store8((T*)e.q_out + (int64_t)gm * e.q_dim + c, v);
      } else if (is_k) {
        T* kp = (T*)e.k_cache + (int64_t)r * e.kv_dim + (c - e.q_dim);
        float rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = Elem<T>::rnd(v[j]);
        if (e.dev_part && r >= e.dev_lo && r < e.dev_hi) {
          float old[8];
          const uint32_t wd[4] = {oldk[p].x, oldk[p].y, oldk[p].z, oldk[p].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            old[2 * j] = __uint_as_float(wd[j] << 16);
            old[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
          }
          if (sf) {
            const float ca[4] = {cd[p].x, cd[p].y, cd[p].z, cd[p].w};
            const float sa[4] = {sd[p].x, sd[p].y, sd[p].z, sd[p].w};
            float rot[8];
            rope_rotate8(old, ca, sa, rot);
#pragma unroll
            for (int j = 0; j < 8; ++j) old[j] = Elem<T>::rnd(rot[j]);
          }
          contrib[p] = dev_add8(rv, old, 0.f);
        }
        store8(kp, rv);
      } else {
        store8((T*)e.v_cache + (int64_t)r * e.kv_dim + (c - e.q_dim - e.kv_dim), v);
      }
    }
  }
  if (k_tile) {
    // fixed-order reduction over the tpr consecutive lanes of each row, the
    // rows' cross-lane steps interleaved so that their latencies overlap
    for (int o = tpr / 2; o > 0; o >>= 1) {
#pragma unroll
      for (int p = 0; p < NP; ++p) contrib[p] += __shfl_xor(contrib[p], o);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int gm = m0 + p * rpp + lr;
      if ((tid % tpr) == 0 && gm < M) e.dev_part[(int64_t)(tn - e.k_tile0) * M + gm] = contrib[p];
    }
  }
}

// Apply the epilogue KIND to a bm x bn fp32 tile held in LDS (row stride cld).
template <typename T, int bm, int bn, int NT, int KIND>
__device__ void run_epilogue(const EpiParams& e, const BOperand& B, const float* Cs, int cld, int m0, int tn,
                             int M, int N, const float* row_scale = nullptr, const ShiftFuse* sf = nullptr) {
  if constexpr (KIND == EPI_QKV && std::is_same<T, bf16_t>::value && (NT % (bn / 8)) == 0) {
    if (e.req.n == 0) {
      qkv_tile_epilogue<T, bm, bn, NT>(e, Cs, cld, m0, tn, M, N, row_scale, sf);
      return;
    }
  }
  constexpr bool swiglu = KIND == EPI_SWIGLU;
  const int cols = swiglu ? bn / 2 : bn;
  const int tpr = cols / 8;  // threads per row (a power of two <= 64 for the QKV deviation reduction)
  const int rpp = NT / tpr;
  const int tid = threadIdx.x;
  if (tid >= rpp * tpr) return;   // idle when tpr does not divide NT (224-wide tiles)
  const int lr = tid / tpr, lc = (tid % tpr) * 8;
  const bool want_dev = KIND == EPI_QKV && e.dev_part != nullptr;
  const int q_end = e.q_dim, k_end = e.q_dim + e.kv_dim;
  const bool k_tile = want_dev && tn * bn < k_end && tn * bn + bn > q_end;
  for (int r0 = 0; r0 < bm; r0 += rpp) {
    const int r = r0 + lr;
    const int gm = m0 + r;
    float contrib = 0.f;
    if (r < bm && gm < M) {
      const float* row = Cs + r * cld;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = row[lc + j];
      if (row_scale) {
        const float rs = row_scale[r];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= rs;
      }
      if constexpr (swiglu) {
        const int f = tn * (bn / 2) + lc;
        if (f < B.n_feat) {
          float u[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) u[j] = row[bn / 2 + lc + j];
          epi_swiglu<T>(e, gm, f, v, u);
        }
      } else {
        const int c = tn * bn + lc;
        if (c < N) {
          if constexpr (KIND == EPI_QKV) contrib = epi_qkv<T>(e, gm, c, v, sf);
          else if constexpr (KIND == EPI_RESID) epi_resid<T>(e, gm, c, v);
          else epi_store<T>(e, gm, c, v);
        }
      }
    }
    if (k_tile) {
      // fixed-order reduction over the tpr consecutive lanes of this row
      for (int o = tpr / 2; o > 0; o >>= 1) contrib += __shfl_xor(contrib, o);
      if ((tid % tpr) == 0 && r < bm && gm < M) e.dev_part[(int64_t)(tn - e.k_tile0) * M + gm] = contrib;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

__device__ __forceinline__ int xcd_remap(int id, int nb) {
  // workgroup id -> tile index so that consecutive tile indices share an XCD
  return (nb & 7) == 0 ? (id & 7) * (nb >> 3) + (id >> 3) : id;
}



// Byte offset of 16-byte chunk c of row r in a swizzled [rows][BK] bf16 tile:
// rows are 128 B, chunk c of row r sits in slot c ^ ((r >> 1) & 7), so the
// 16 rows read by one fragment load cover all 64 banks exactly once.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

#ifndef CB_GEMM_NSTAGE
#define CB_GEMM_NSTAGE 4
#endif
#ifndef CB_GEMM_MINBLOCKS
#define CB_GEMM_MINBLOCKS 1
#endif
#ifndef CB_GEMM_ILV
#define CB_GEMM_ILV 1
#endif
constexpr int NSTAGE = CB_GEMM_NSTAGE;          // LDS ring depth (K steps in flight)
constexpr int kStageBytes = (BM + BN) * BK * 2;  // 32 KB
// the ring, or the fp32 tile plus the folded RMSNorm's half sums and row scales
constexpr int kGemmSmem3 =
    NSTAGE * kStageBytes > BM * CLD * 4 + 3 * BM * 4 ? NSTAGE * kStageBytes : BM * CLD * 4 + 3 * BM * 4;

// Re-alignment part of a fused QKV launch: workgroup b of sf.n_wg rotates
// the keys of its share of rows [row0, row1) that are not in s_in, 16
// elements per thread as rope_shift_kernel does (the same rotation and
// rounding).  The recomputed rows are marked in LDS first: their keys are
// replaced by the projection's epilogue in the same launch.
__device__ __forceinline__ void shift_part(const ShiftFuse& sf, int b, char* smem) {
  const int tid = threadIdx.x;
  const int per = (sf.row1 - sf.row0 + sf.n_wg - 1) / sf.n_wg;
  const int r_lo = sf.row0 + b * per, r_hi = min(sf.row1, r_lo + per);
  if (r_lo >= r_hi) return;   // uniform over the workgroup
  unsigned char* skip = (unsigned char*)smem;
  for (int i = tid; i < r_hi - r_lo; i += 256) skip[i] = 0;
  __syncthreads();
  for (int i = tid; i < sf.m_in; i += 256) {
    const int r = sf.s_in[i];
    if (r >= r_lo && r < r_hi) skip[r - r_lo] = 1;
  }
  __syncthreads();
  const int upr = sf.kv_dim / 16;   // 16-element units per row
  const int n_units = (r_hi - r_lo) * upr;
  for (int u = tid; u < n_units; u += 256) {
    const int rr = u / upr;
    if (skip[rr]) continue;
    const int r = r_lo + rr;
    const int delta = chunk_delta_scan(sf.offs, sf.n_chunks, r);
    bf16_t* p = (bf16_t*)sf.k + (int64_t)r * sf.kv_dim + (u % upr) * 16;
    float v[2][8];
    load8(p, v[0]);
    load8(p + 8, v[1]);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int e = ((u % upr) * 16 + x * 8) % sf.hd;
      const int64_t t = (int64_t)delta * (sf.hd / 2) + e / 2;
      float o[8];
      rope_rotate8(v[x], sf.cos + t, sf.sin + t, o);
      store8(p + x * 8, o);
    }
  }
}

struct NoShift {};

// 128x128 output tiles.  With SX = ShiftFuse (the QKV projection with the
// layer's re-alignment in the same launch) the first sx.n_wg workgroups
// shift keys, on CUs the projection's tiles leave idle, and the rest are
// the projection's tiles.
template <int KIND, typename SX>
__global__ __launch_bounds__(256, CB_GEMM_MINBLOCKS) void gemm_bf16_kernel(GemmArgs g, int mt, int ntiles, SX sx) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmSmem3];
  constexpr bool kShift = std::is_same<SX, ShiftFuse>::value;
  static_assert(!kShift || KIND == EPI_QKV, "only the QKV projection re-aligns");
  const ShiftFuse* sf = nullptr;
  int bid = blockIdx.x, nblk = gridDim.x;
  if constexpr (kShift) {
    if (bid < sx.n_wg) {
      shift_part(sx, bid, smem);
      return;
    }
    bid -= sx.n_wg;
    nblk -= sx.n_wg;
    sf = &sx;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = xcd_remap(bid, nblk);
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * BM;
  const int M = g.M, K = g.K;
  const int kchunk = ((K + g.splits - 1) / g.splits + BK - 1) / BK * BK;
  const int kb = blockIdx.y * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  // DMA plan: wave w moves row groups (w*4 + j)*8 .. +7 of the A and B tiles
  // (j = 0..3); lane i of a group fills slot i%8 of row i/8 with the logical
  // chunk slot ^ ((row >> 1) & 7).  Rows past the matrix and chunks past the
  // K range are out of the buffer's range and load as zero.
  const uint32_t kOOB = 0x80000000u;
  // folded RMSNorm (QKV only): A rows gathered from the un-normalised input
  const bool fold = KIND == EPI_QKV && g.a_norm;
  const int a_rows_total = fold ? g.a_src_rows : M;
  __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)a_rows_total * K * 2));
  __amdgpu_buffer_rsrc_t rb[4];
  uint32_t aoff[4], boff[4];
  int lcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int grp = w * 4 + j;
    const int row = grp * 8 + (lane >> 3);
    const int slot = lane & 7;
    lcol[j] = (slot ^ ((row >> 1) & 7)) * 8;      // logical k offset of this lane's chunk
    int src = m0 + row;
    if (fold && src < M && g.a_rows) src = g.a_rows[src];
    aoff[j] = (m0 + row < M && src >= 0 && src < a_rows_total) ? (uint32_t)((int64_t)src * K * 2) : kOOB;
    // B: the 8 rows of a group always come from one weight matrix
    const int r0 = grp * 8;
    const void* base;
    int brow, nrows;
    if (g.B.mode == 0) {
      const int c0 = tn * BN + r0;
      if (c0 < g.B.n1) { base = g.B.p0; brow = c0; nrows = g.B.n1; }
      else if (c0 < g.B.n2) { base = g.B.p1; brow = c0 - g.B.n1; nrows = g.B.n2 - g.B.n1; }
      else { base = g.B.p2; brow = c0 - g.B.n2; nrows = g.N - g.B.n2; }
    } else {
      base = r0 < BN / 2 ? g.B.p0 : g.B.p1;
      brow = tn * (BN / 2) + (r0 % (BN / 2));
      nrows = g.B.n_feat;
    }
    rb[j] = make_rsrc(base, (uint32_t)((int64_t)(nrows > 0 ? nrows : 0) * K * 2));
    const int myrow = brow + (lane >> 3);
    boff[j] = myrow < nrows ? (uint32_t)((int64_t)myrow * K * 2) : kOOB;
  }

  auto issue_group = [&](int stage, int k0, int j) {
    char* sa = smem + stage * kStageBytes;
    char* sb = sa + BM * BK * 2;
    const int grp = w * 4 + j;
    const int kk = k0 + lcol[j];
    const bool kin = kk < ke;
    const uint32_t oa = (kin && aoff[j] != kOOB) ? aoff[j] + kk * 2 : kOOB;
    const uint32_t ob = (kin && boff[j] != kOOB) ? boff[j] + kk * 2 : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + grp * 1024), 16, oa, 0, 0, CB_A_AUX);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[j], (lds_void*)(sb + grp * 1024), 16, ob, 0, 0, CB_W_AUX);
  };
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_group(stage, k0, j);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int fr = lane & 15, fc = lane >> 4;
  // folded RMSNorm: the two waves that share rows wm .. wm+63 split the sum
  // of squares of those rows: wave w adds, for the 32-deep half ks = w & 1 of
  // every step, the Gram block A_i A_i^T of each of its 16-row fragments on
  // the matrix cores (its diagonal holds the rows' sums of squares); the
  // fragments are the ones the step's products already use
  f32x4_t gram[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) gram[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool do_ssq = fold;

  // one step's MFMAs; with CB_GEMM_ILV the next stage's DMA (nstage >= 0) is
  // issued one row group at a time between them
  auto compute = [&](int stage, int nstage, int nk0) {
    const char* sa = smem + stage * kStageBytes;
    const char* sb = sa + BM * BK * 2;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + swz(wm + i * 16 + fr, ks * 4 + fc));
        bfr[i] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn + i * 16 + fr, ks * 4 + fc));
      }
      if (do_ssq && ks == (w & 1)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gram[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], af[i], gram[i], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
#if CB_GEMM_ILV
        const int slot = ks * 4 + i;   // 8 slots per step, 4 row groups to issue
        if (nstage >= 0 && (slot & 1)) {
          __builtin_amdgcn_sched_barrier(0);
          issue_group(nstage, nk0, slot >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
#endif
      }
    }
  };

  // prologue: NSTAGE-1 K steps in flight
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < nk) issue(st, kb + st * BK);
  // main loop, unrolled by the ring depth so every LDS address is static
  for (int it0 = 0; it0 < nk; it0 += NSTAGE) {
#pragma unroll
    for (int u = 0; u < NSTAGE; ++u) {
      const int it = it0 + u;
      if (it < nk) {
        // this wave's DMA for step `it` is done once at most the later
        // steps' 8 loads per step are outstanding
        const int later = min(nk - 1 - it, NSTAGE - 2);
        static_assert(NSTAGE <= 5, "wait counts below cover at most three later steps");
        if (later >= 3) CB_WAIT_VMCNT(24);
        else if (later == 2) CB_WAIT_VMCNT(16);
        else if (later == 1) CB_WAIT_VMCNT(8);
        else CB_WAIT_VMCNT(0);
        CB_BARRIER();   // every wave's step `it` is in LDS; step it-1's buffer is free
        const bool more = it + NSTAGE - 1 < nk;
#if CB_GEMM_ILV
        compute(u, more ? (u + NSTAGE - 1) % NSTAGE : -1, kb + (it + NSTAGE - 1) * BK);
#else
        if (more) issue((u + NSTAGE - 1) % NSTAGE, kb + (it + NSTAGE - 1) * BK);
        compute(u, -1, 0);
#endif
      }
    }
  }
  CB_WAIT_VMCNT(0);
  __syncthreads();

  // folded RMSNorm: each wave's half of a row's sum of squares after the
  // accumulator tile, then the row scales 1 / sqrt(mean(x^2) + eps) from the
  // two halves in a fixed order
  float* rhalf = (float*)(smem + BM * CLD * 4);   // [2][BM]
  float* rscale = rhalf + 2 * BM;                  // [BM]
  if (do_ssq) {
    // diagonal element (r, r) of a 16x16 block: lane r + 16 (r / 4), slot r % 4
    const int r = fr;
    if (lane == r + 16 * (r >> 2)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rhalf[(w & 1) * BM + wm + i * 16 + r] = gram[i][r & 3];
    }
  }

  // accumulators -> fp32 tile in LDS.  Lane l of a 16x16 block holds column
  // l%16 and rows 4*(l/16) .. 4*(l/16)+3.
  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        Cs[(wm + i * 16 + fc * 4 + v) * CLD + wn + j * 16 + fr] = acc[i][j][v];
  __syncthreads();
  if (fold) {
    if (tid < BM) rscale[tid] = 1.0f / sqrtf((rhalf[tid] + rhalf[BM + tid]) / (float)K + g.a_eps);
    __syncthreads();
  }

  if (g.splits > 1) {
    // split-K partial; splitk_epilogue_kernel adds the splits in order
    const int ldp = ntiles * BN;
    float* P = g.part + (int64_t)blockIdx.y * M * ldp;
    for (int idx = tid; idx < BM * BN / 4; idx += 256) {
      const int r = idx / (BN / 4), c4 = (idx % (BN / 4)) * 4;
      if (m0 + r < M)
        *reinterpret_cast<float4*>(P + (int64_t)(m0 + r) * ldp + tn * BN + c4) =
            *reinterpret_cast<const float4*>(Cs + r * CLD + c4);
    }
    return;
  }
  run_epilogue<bf16_t, BM, BN, 256, KIND>(g.epi, g.B, Cs, CLD, m0, tn, M, g.N, fold ? rscale : nullptr, sf);
}


// ---------------------------------------------------------------------------
// bf16 MFMA kernel, large tile for the gate/up projection: 256 rows x LBN
// columns (LBN/2 gate + LBN/2 up features) with 8 waves, K step 32 with a
// 4-deep LDS ring.  The tile halves the L2-to-LDS bytes per flop of the
// 128x128 kernel.  LBN = 224 gives the 8B layer's 493 rows x 14336 features
// 2 x 128 = 256 workgroups, one per CU (256 wide leaves 32 CUs idle); its
// waves are 4 (M) x 2 (N) of 64x112 (4x7 MFMA blocks); LBN = 256 uses
// 2 x 4 waves of 128x64.
// ---------------------------------------------------------------------------
#ifndef CB_BIG_BN
#define CB_BIG_BN 256
#endif
#ifndef CB_BIG_WAVES
#define CB_BIG_WAVES 8
#endif
#ifndef CB_BIG_NSTAGE
#define CB_BIG_NSTAGE 4
#endif
// gate/up on the software-pipelined four-wave kernel instead
#ifndef CB_GATEUP_W4
#define CB_GATEUP_W4 1
#endif
constexpr int LBM = 256, LBN = CB_BIG_BN, LBK = 32, LNS = CB_BIG_NSTAGE, LCLD = LBN + 4;
constexpr int kLW = CB_BIG_WAVES;                    // waves per workgroup
static_assert(LBN == 224 || LBN == 256, "large tile: 224 or 256 columns");
static_assert(kLW == 8 || (kLW == 4 && LBN == 256), "8 waves, or 4 waves of 128x128");
constexpr int kLNT = 64 * kLW;
constexpr int kLWN = kLW == 4 ? 2 : (LBN == 224 ? 2 : 4);   // waves along N
constexpr int kLWTM = LBM / (kLW / kLWN);            // wave tile rows (64 or 128)
constexpr int kLWTN = LBN / kLWN;                    // wave tile columns (112, 64 or 128)
constexpr int kLFA = kLWTM / 16, kLFB = kLWTN / 16;  // MFMA blocks per wave
constexpr int kLStage = (LBM + LBN) * LBK * 2;       // 30 or 32 KB
static_assert(LNS >= 2 && LNS <= 5 && LNS * kLStage <= 160 * 1024, "ring depth");
constexpr int kLSmem = LNS * kLStage > 128 * LCLD * 4 ? LNS * kLStage : 128 * LCLD * 4;
static_assert(LBK == kGateupStep, "the packed gate/up layout follows the large kernel's K step");
constexpr int kLBlocksA = LBM / 16, kLBlocks = (LBM + LBN) / 16;   // 1 KB blocks per stage
constexpr int kLBPW = (kLBlocks + kLW - 1) / kLW;   // blocks per wave (at most)
static_assert(kLBPW <= 8 && kLFA % kLBPW == 0, "blocks are issued between MFMA rows");

// 64-byte rows (BK = 32) in 1 KB blocks of 16 rows.  Inside a block, row r
// sits in row slot rho(r) and its 16-byte chunk c in slot c ^ ((r >> 1) & 3).
// A fragment load (rows r = 0..15 of a block, chunk = lane / 16) then lands
// on the same 16-byte bank groups, lane by lane, as the 128-byte-row layout
// of the 128x128 kernel, which measures free of bank conflicts; the plain
// (r >> 2) XOR of 64-byte rows measured two-way conflicts on gfx950.
__device__ __forceinline__ int rho16(int r) { return 4 * ((r >> 1) & 3) + 2 * (r & 1) + ((r >> 3) & 1); }
__device__ __forceinline__ int rho16_inv(int s) { return ((s & 1) << 3) | ((s >> 2) << 1) | ((s >> 1) & 1); }
__device__ __forceinline__ int swz32(int r, int c) {
  const int rl = r & 15;
  return (r >> 4) * 1024 + rho16(rl) * 64 + ((c ^ ((rl >> 1) & 3)) << 4);
}

// s_waitcnt with the later steps' loads still allowed in flight (ps loads per
// step, later <= 4 steps)
#define CB_WAIT_LATER(ps, later)                 \
  do {                                           \
    if ((later) >= 4) CB_WAIT_VMCNT(4 * (ps));   \
    else if ((later) == 3) CB_WAIT_VMCNT(3 * (ps)); \
    else if ((later) == 2) CB_WAIT_VMCNT(2 * (ps)); \
    else if ((later) == 1) CB_WAIT_VMCNT(ps);    \
    else CB_WAIT_VMCNT(0);                       \
  } while (0)

template <int KIND>
__global__ __launch_bounds__(kLNT, 1) void gemm_bf16_big_kernel(GemmArgs g, int mt, int ntiles) {
  __shared__ __attribute__((aligned(16))) char smem[kLSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * LBM;
  const int M = g.M, K = g.K;
  const int nk = (K + LBK - 1) / LBK;

  // DMA plan: a wave instruction fills one 1 KB block of 16 rows x 64 B;
  // wave w moves blocks w, w + kLW, w + 2 kLW, ... of the stage (A's blocks
  // first, then B's).
  const uint32_t kOOB = 0x80000000u;
  const int nbw = (kLBlocks - w + kLW - 1) / kLW;   // blocks of this wave (uniform)
  const int rl = rho16_inv(lane >> 2);      // the row whose slot this lane fills
  const int lcol = ((lane & 3) ^ ((rl >> 1) & 3)) * 8;
  __amdgpu_buffer_rsrc_t rs[kLBPW];
  uint32_t off[kLBPW];
  int dst[kLBPW];
  // packed gate/up operand: block (tile tn, step s) starts at
  // (tn * nk + s) * LBN * 64 bytes; off[] then holds the lane's byte offset
  // inside the block
  const bool packed = LBN == kGateupTile && g.B.mode == 1 && g.B.packed != nullptr;
#pragma unroll
  for (int j = 0; j < kLBPW; ++j) {
    const int blk = min(w + kLW * j, kLBlocks - 1);
    if (blk >= kLBlocksA && packed) {
      const int r0 = (blk - kLBlocksA) * 16;
      rs[j] = make_rsrc(g.B.packed, (uint32_t)pack_gateup_bytes(g.B.n_feat, K));
      off[j] = (uint32_t)((r0 + rl) * 64 + lcol * 2);
      dst[j] = blk * 1024;
    } else if (blk < kLBlocksA) {
      const int row = blk * 16 + rl;
      rs[j] = make_rsrc(g.A, (uint32_t)((int64_t)M * K * 2));
      off[j] = m0 + row < M ? (uint32_t)((int64_t)(m0 + row) * K * 2) : kOOB;
      dst[j] = blk * 1024;
    } else {
      const int r0 = (blk - kLBlocksA) * 16;
      const void* base;
      int brow, nrows;
      if (g.B.mode == 0) {
        const int c0 = tn * LBN + r0;
        if (c0 < g.B.n1) { base = g.B.p0; brow = c0; nrows = g.B.n1; }
        else if (c0 < g.B.n2) { base = g.B.p1; brow = c0 - g.B.n1; nrows = g.B.n2 - g.B.n1; }
        else { base = g.B.p2; brow = c0 - g.B.n2; nrows = g.N - g.B.n2; }
      } else {
        base = r0 < LBN / 2 ? g.B.p0 : g.B.p1;
        brow = tn * (LBN / 2) + (r0 % (LBN / 2));
        nrows = g.B.n_feat;
      }
      rs[j] = make_rsrc(base, (uint32_t)((int64_t)(nrows > 0 ? nrows : 0) * K * 2));
      const int myrow = brow + rl;
      off[j] = myrow < nrows ? (uint32_t)((int64_t)myrow * K * 2) : kOOB;
      dst[j] = blk * 1024;   // B's blocks follow A's in the stage
    }
  }
  auto issue_group = [&](int stage, int k0, int j) {
    if (j >= nbw) return;
    uint32_t o;
    if (packed && w + kLW * j >= kLBlocksA) {
      o = (uint32_t)((tn * nk + k0 / LBK) * (LBN * 64)) + off[j];
    } else {
      const int kk = k0 + lcol;
      o = (kk < K && off[j] != kOOB) ? off[j] + kk * 2 : kOOB;
    }
    static_assert(kLBlocksA % kLW == 0, "block w + kLW j is a weight block exactly when kLW j >= kLBlocksA");
    if (kLW * j >= kLBlocksA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[j], (lds_void*)(smem + stage * kLStage + dst[j]), 16, o, 0, 0,
                                               CB_W_AUX);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[j], (lds_void*)(smem + stage * kLStage + dst[j]), 16, o, 0, 0,
                                               CB_A_AUX);
  };
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < kLBPW; ++j) issue_group(stage, k0, j);
  };

  f32x4_t acc[kLFA][kLFB];
#pragma unroll
  for (int i = 0; i < kLFA; ++i)
#pragma unroll
    for (int j = 0; j < kLFB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wm = (w / kLWN) * kLWTM, wn = (w % kLWN) * kLWTN;
  const int fr = lane & 15, fc = lane >> 4;
  // one step's MFMAs, with the next stage's loads (nstage >= 0) issued one
  // block at a time between the MFMA rows instead of in one burst
  auto compute = [&](int stage, int nstage, int nk0) {
    const char* sa = smem + stage * kLStage;
    const char* sb = sa + LBM * LBK * 2;
    bf16x8_t af[kLFA], bfr[kLFB];
#pragma unroll
    for (int i = 0; i < kLFA; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(sa + swz32(wm + i * 16 + fr, fc));
#pragma unroll
    for (int j = 0; j < kLFB; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + swz32(wn + j * 16 + fr, fc));
#pragma unroll
    for (int i = 0; i < kLFA; ++i) {
#pragma unroll
      for (int j = 0; j < kLFB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      constexpr int per = kLFA / kLBPW;   // MFMA rows between issued blocks
      if (nstage >= 0 && i % per == per - 1) {
        __builtin_amdgcn_sched_barrier(0);
        issue_group(nstage, nk0, i / per);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

#pragma unroll
  for (int st = 0; st < LNS - 1; ++st)
    if (st < nk) issue(st, st * LBK);
  for (int it0 = 0; it0 < nk; it0 += LNS) {
#pragma unroll
    for (int u = 0; u < LNS; ++u) {
      const int it = it0 + u;
      if (it < nk) {
        // this wave's step `it` landed once at most the later steps' loads
        // (nbw per step) are outstanding; then every wave's have (barrier)
        const int later = min(nk - 1 - it, LNS - 2);
        if (nbw == kLBPW) CB_WAIT_LATER(kLBPW, later);
        else CB_WAIT_LATER(kLBPW - 1, later);
        CB_BARRIER();
        const bool more = it + LNS - 1 < nk;
        compute(u, more ? (u + LNS - 1) % LNS : -1, (it + LNS - 1) * LBK);
      }
    }
  }
  CB_WAIT_VMCNT(0);
  __syncthreads();

  // epilogue in two halves of 128 rows (the fp32 tile of 256 rows does not fit)
  float* Cs = (float*)smem;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm / 128 == half) {
#pragma unroll
      for (int i = 0; i < kLFA; ++i)
#pragma unroll
        for (int j = 0; j < kLFB; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            Cs[(wm - half * 128 + i * 16 + fc * 4 + v) * LCLD + wn + j * 16 + fr] = acc[i][j][v];
    }
    __syncthreads();
    run_epilogue<bf16_t, 128, LBN, kLNT, KIND>(g.epi, g.B, Cs, LCLD, m0 + half * 128, tn, M, g.N);
    __syncthreads();
  }
}

// Four waves of 128 x 128 on the 256 x 256 gate/up tile (one wave per SIMD),
// software-pipelined: in the step for K step `it` a wave first issues the
// LDS fragment reads of step it + 1 (into the other register set), then the
// 64 MFMAs of step it from the fragments read one step earlier, with the
// direct-to-LDS loads of step it + 3 between the MFMA rows.  The barrier at
// the top of a step therefore waits for step it + 1's loads, and the LDS
// reads never stand between a barrier and the matrix cores.  Per step and
// CU this moves 64 KB of fragment reads and 32 KB of loads through LDS
// against 96 KB + 32 KB for eight waves of 128 x 64.
// TBN = kGateupTile columns: 256, or 224 (the 8B layer's 14336 features then
// make 2 x 128 = 256 workgroups, one per CU; its waves are 128 x 112 and a
// stage's two missing B blocks are loads past the buffer's end into padding).
template <int KIND>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4_kernel(GemmArgs g, int mt, int ntiles) {
  constexpr int TBN = kGateupTile, NS = 4, CLD = TBN + 4;
  constexpr int FB = TBN / 32;                                   // B fragments per wave (8 or 7)
  constexpr int kStage = (LBM + 256) * LBK * 2;                 // 32 KB (padded for TBN = 224)
  constexpr int kSmem = NS * kStage > 128 * CLD * 4 ? NS * kStage : 128 * CLD * 4;
  constexpr int kBlocksA = LBM / 16;                             // 16 A blocks, then TBN/16 B blocks
  constexpr int kBlocks = kBlocksA + TBN / 16;
  static_assert(TBN == 256 || TBN == 224, "gate/up tile width");
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * LBM;
  const int M = g.M, K = g.K;
  const int nk = K / LBK;   // whole steps (checked by the host)

  // DMA plan: wave w fills blocks w + 4 j (j < 8) of a stage: A blocks for
  // j < 4, B blocks for j >= 4.  A block's byte offset for the step at k0 is
  // base[j] + k0 * mul[j] (2 bytes per element of a row-major operand; one
  // 16 KB block per step in the packed layout); rows past the operand start
  // past the buffer's end and load as zero, so the main loop has no branch.
  const uint32_t kOOB = 0x80000000u;
  const int rl = rho16_inv(lane >> 2);
  const int lcol = ((lane & 3) ^ ((rl >> 1) & 3)) * 8;
  const bool packed = g.B.mode == 1 && g.B.packed != nullptr;
  __amdgpu_buffer_rsrc_t rs[8];
  uint32_t base[8];
  int mul[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int blk = w + 4 * j;
    if (blk < kBlocksA && g.a_packed) {
      // A in the step-major layout: one 16 KB block per (row tile, step);
      // the padded rows of the last tile only feed output rows past M
      const int row = blk * 16 + rl;
      rs[j] = make_rsrc(g.A, (uint32_t)((int64_t)act_packed_rows(M) * K * 2));
      base[j] = (uint32_t)(tm * nk) * (LBM * 64) + (uint32_t)(row * 64 + lcol * 2);
      mul[j] = LBM * 64 / LBK;
    } else if (blk < kBlocksA) {
      const int row = blk * 16 + rl;
      rs[j] = make_rsrc(g.A, (uint32_t)((int64_t)M * K * 2));
      base[j] = (m0 + row < M ? (uint32_t)((int64_t)(m0 + row) * K * 2) : kOOB) + lcol * 2;
      mul[j] = 2;
    } else if (blk >= kBlocks) {
      // padding block of a 224-wide tile: a load past every buffer (zeros)
      rs[j] = make_rsrc(g.A, 0u);
      base[j] = kOOB;
      mul[j] = 0;
    } else if (packed) {
      const int r0 = (blk - kBlocksA) * 16;
      rs[j] = make_rsrc(g.B.packed, (uint32_t)pack_gateup_bytes(g.B.n_feat, K));
      base[j] = (uint32_t)(tn * nk) * (TBN * 64) + (uint32_t)((r0 + rl) * 64 + lcol * 2);
      mul[j] = TBN * 64 / LBK;
    } else {
      const int r0 = (blk - kBlocksA) * 16;
      const int f = tn * (TBN / 2) + (r0 % (TBN / 2)) + rl;
      // B blocks 0..7 of the tile are gate rows, 8..15 up rows
      rs[j] = make_rsrc(r0 < TBN / 2 ? g.B.p0 : g.B.p1, (uint32_t)((int64_t)g.B.n_feat * K * 2));
      base[j] = (f < g.B.n_feat ? (uint32_t)((int64_t)f * K * 2) : kOOB) + lcol * 2;
      mul[j] = 2;
    }
  }
  // a step past the last one loads zeros (offset past every buffer) into a
  // stage that is never read again, so the issue needs no branch either
  auto issue_block = [&](int stage, int k0, int j) {
    const uint32_t o = (base[j] + (uint32_t)(k0 * mul[j])) | ((uint32_t)(k0 >= K) << 31);
    if (j < 4)   // blocks w + 4 j < 16: activation rows
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[j], (lds_void*)(smem + stage * kStage + (w + 4 * j) * 1024), 16, o,
                                               0, 0, CB_A_AUX);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[j], (lds_void*)(smem + stage * kStage + (w + 4 * j) * 1024), 16, o,
                                               0, 0, CB_W_AUX);
  };

  f32x4_t acc[8][FB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // the 256 accumulator registers live in the AGPR file (an empty asm
      // statement with an AGPR operand places them there), which leaves the
      // 256 VGPRs to the two fragment sets and the addressing
      asm volatile("" : "+a"(acc[i][j]));
    }
  const int wm = (w >> 1) * 128, wn = (w & 1) * (TBN / 2);
  const int fr = lane & 15, fc = lane >> 4;
  bf16x8_t fa[2][8], fb[2][FB];
  auto read_frags = [&](int stage, int set) {
    const char* sa = smem + stage * kStage;
    const char* sb = sa + LBM * LBK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[set][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz32(wm + i * 16 + fr, fc));
#pragma unroll
    for (int j = 0; j < FB; ++j) fb[set][j] = *reinterpret_cast<const bf16x8_t*>(sb + swz32(wn + j * 16 + fr, fc));
  };

  // prologue: steps 0..NS-1 in flight, step 0's fragments in set 0
#pragma unroll
  for (int st = 0; st < NS; ++st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_block(st, st * LBK, j);
  }
  CB_WAIT_VMCNT(8 * (NS - 1));
  CB_BARRIER();
  read_frags(0, 0);

  // main loop, unrolled by the ring depth so every LDS address and register
  // set is static (the host launches this kernel only when NS divides the
  // step count).  Step it's stage is free once every wave has read its
  // fragments (during step it - 1, complete at the barrier of step it), so
  // step it + NS is loaded into it from then on: NS steps in flight.
  for (int it0 = 0; it0 < nk; it0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int it = it0 + u;
      const int cur = u & 1;   // NS is even: the fragment set of step it is it & 1
      // this wave's loads of step it + 1 landed once only those of steps
      // it + 2 .. it + NS - 1 are outstanding; then every wave's have (barrier)
      CB_WAIT_VMCNT(8 * (NS - 2));
      CB_BARRIER();
      // the next step's fragments (past the last step: unused) are read two
      // at a time between the MFMA rows, so the four waves' reads do not
      // queue up at the LDS in front of their first MFMAs
      const char* na = smem + ((u + 1) % NS) * kStage;
      const char* nb = na + LBM * LBK * 2;
      const int nk0 = (it + NS) * LBK;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < FB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fa[cur ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(na + swz32(wm + i * 16 + fr, fc));
        if (i < FB) fb[cur ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(nb + swz32(wn + i * 16 + fr, fc));
        issue_block(u, nk0, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  CB_WAIT_VMCNT(0);
  __syncthreads();

  // epilogue in two halves of 128 rows
  float* Cs = (float*)smem;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm / 128 == half) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) Cs[(i * 16 + fc * 4 + v) * CLD + wn + j * 16 + fr] = acc[i][j][v];
    }
    __syncthreads();
    run_epilogue<bf16_t, 128, TBN, 256, KIND>(g.epi, g.B, Cs, CLD, m0 + half * 128, tn, M, g.N);
    __syncthreads();
  }
}

// Split-K finish: one thread per 8 output columns of a row adds the split
// partials in split order straight from memory and applies the epilogue.
// 16 rows x one 128-column tile per workgroup; no LDS staging.
template <int KIND>
__device__ __forceinline__ float sum8(const GemmArgs& g, int ldp, int gm, int col, float v[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.f;
  for (int sp = 0; sp < g.splits; ++sp) {
    const float* p = g.part + ((int64_t)sp * g.M + gm) * ldp + col;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  return 0.f;
}

template <int KIND>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(GemmArgs g, int ntiles) {
  const int tn = blockIdx.y;
  const int ldp = ntiles * BN;
  const int tid = threadIdx.x;
  const EpiParams& e = g.epi;
  constexpr bool swiglu = KIND == EPI_SWIGLU;
  constexpr int cols = swiglu ? BN / 2 : BN;
  constexpr int tpr = cols / 8;
  constexpr int rpb = 256 / tpr;
  const int r = blockIdx.x * rpb + tid / tpr;
  const int lc = (tid % tpr) * 8;
  const int gm = r;
  const bool k_tile = KIND == EPI_QKV && e.dev_part != nullptr && tn * BN < e.q_dim + e.kv_dim &&
                      tn * BN + BN > e.q_dim;
  float contrib = 0.f;
  if (gm < g.M) {
    float v[8];
    sum8<KIND>(g, ldp, gm, tn * BN + lc, v);
    if constexpr (swiglu) {
      float u[8];
      sum8<KIND>(g, ldp, gm, tn * BN + BN / 2 + lc, u);
      const int f = tn * (BN / 2) + lc;
      if (f < g.B.n_feat) epi_swiglu<bf16_t>(e, gm, f, v, u);
    } else {
      const int c = tn * BN + lc;
      if (c < g.N) {
        if constexpr (KIND == EPI_QKV) contrib = epi_qkv<bf16_t>(e, gm, c, v, nullptr);
        else if constexpr (KIND == EPI_RESID) epi_resid<bf16_t>(e, gm, c, v);
        else epi_store<bf16_t>(e, gm, c, v);
      }
    }
  }
  if (k_tile) {
    for (int o = tpr / 2; o > 0; o >>= 1) contrib += __shfl_xor(contrib, o);
    if ((tid % tpr) == 0 && gm < g.M) e.dev_part[(int64_t)(tn - e.k_tile0) * g.M + gm] = contrib;
  }
}

// Split-K finish of a residual projection fused with the RMSNorm that follows
// it (attention output projection -> h -> RMSNorm -> the MLP input): one
// 256-thread workgroup per row; every thread owns the same 8-column groups as
// rmsnorm_kernel and adds in the same order, so h and the normalised row are
// bit-identical to the two kernels run one after the other.
constexpr int kResidNormGroups = 4;  // 8-column groups per thread: rows up to 256 * 8 * 4 = 8192 wide

__global__ __launch_bounds__(256) void resid_norm_kernel(GemmArgs g, int ntiles, const float* __restrict__ gain,
                                                         float eps, bf16_t* __restrict__ hn, int hn_packed) {
  __shared__ float red[4];
  const int gm = blockIdx.x;
  const int ldp = ntiles * BN;
  const int d = g.N;
  const EpiParams& e = g.epi;
  const int r = map_row(gm, e.rmap1, e.rmap2);
  float* hrow = (float*)e.out + (int64_t)gm * d;
  float h[kResidNormGroups][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kResidNormGroups; ++i) {
    const int c = (threadIdx.x + i * 256) * 8;
    if (c < d) {
      float v[8], x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      sum8<EPI_RESID>(g, ldp, gm, c, v);
      if (r >= 0 && r < e.T) {
        if (e.resid_f32) load8((const float*)e.resid + (int64_t)r * d + c, x);
        else load8((const bf16_t*)e.resid + (int64_t)r * d + c, x);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[i][j] = x[j] + v[j];  // h = residual + projection (fp32)
        ss += h[i][j] * h[i][j];
      }
      store8(hrow + c, h[i]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int i = 0; i < kResidNormGroups; ++i) {
    const int c = (threadIdx.x + i * 256) * 8;
    if (c < d) {
      float gg[8], o[8];
      load8(gain + c, gg);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (h[i][j] / rs) * gg[j];
      store8(hn + (hn_packed ? act_packed_index(gm, c, d) : (int64_t)gm * d + c), o);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT kernel
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, int mt, int ntiles) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  __shared__ __attribute__((aligned(16))) float Cs[FBM * FCLD];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x % mt, tn = blockIdx.x / mt;
  const int m0 = tm * FBM, M = g.M, K = g.K;
  const int ty = tid / 16, tx = tid % 16;
  const float* A = (const float*)g.A;
  // loader: 4 A and 4 B elements per thread per K step
  const float* bptr[4];
  int lrow[4], lk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    lrow[i] = c / FBK;
    lk[i] = c % FBK;
    bptr[i] = b_row<float>(g.B, K, g.N, tn, FBN, lrow[i]);
  }
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + lk[i];
      const int gm = m0 + lrow[i];
      As[lk[i]][lrow[i]] = (gm < M && k < K) ? A[(int64_t)gm * K + k] : 0.f;
      Bs[lk[i]][lrow[i]] = (bptr[i] && k < K) ? bptr[i][k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FBK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Cs[(ty * 4 + i) * FCLD + tx * 4 + j] = acc[i][j];
  __syncthreads();
  switch (g.epi.kind) {
    case EPI_QKV: run_epilogue<float, FBM, FBN, 256, EPI_QKV>(g.epi, g.B, Cs, FCLD, m0, tn, M, g.N); break;
    case EPI_RESID: run_epilogue<float, FBM, FBN, 256, EPI_RESID>(g.epi, g.B, Cs, FCLD, m0, tn, M, g.N); break;
    case EPI_SWIGLU: run_epilogue<float, FBM, FBN, 256, EPI_SWIGLU>(g.epi, g.B, Cs, FCLD, m0, tn, M, g.N); break;
    default: run_epilogue<float, FBM, FBN, 256, EPI_STORE>(g.epi, g.B, Cs, FCLD, m0, tn, M, g.N); break;
  }
}

}  // namespace

int gemm_bn(int dtype) { return dtype == CB_BF16 ? BN : FBN; }



int gemm_n_tiles(int dtype, const BOperand& B, int N) {
  const int bn = gemm_bn(dtype);
  if (B.mode == 1) return (B.n_feat + bn / 2 - 1) / (bn / 2);
  return (N + bn - 1) / bn;
}

#ifndef CB_SPLIT_TILES
#define CB_SPLIT_TILES 48
#endif
int gemm_splits(int dtype, int n_tiles, int K) {
  if (dtype != CB_BF16) return 1;
  int s = 1;
  while (s < 4 && n_tiles * s < CB_SPLIT_TILES && K / (2 * s) >= 1024) s *= 2;
  return s;
}

namespace {

// one thread per 16-byte chunk of the packed operand
__global__ __launch_bounds__(256) void pack_gateup_kernel(const bf16_t* __restrict__ gate,
                                                          const bf16_t* __restrict__ up, int n_feat, int K, int nk,
                                                          int64_t n_chunks, u32x4_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_chunks) return;
  const int c = (int)(q & 3);                                  // 16-byte chunk of a 64-byte row step
  const int r = (int)((q >> 2) % kGateupTile);                 // row of the tile
  const int64_t ts = (q >> 2) / kGateupTile;                   // tile * nk + step
  const int step = (int)(ts % nk), tile = (int)(ts / nk);
  const int f = tile * (kGateupTile / 2) + (r % (kGateupTile / 2));
  const int col = step * kGateupStep + c * 8;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (f < n_feat && col < K) {
    const bf16_t* src = (r < kGateupTile / 2 ? gate : up) + (int64_t)f * K + col;
    v = *reinterpret_cast<const u32x4_t*>(src);
  }
  out[q] = v;
}

}  // namespace

namespace {

// one thread per 8 elements of a row of [W_q; W_k; W_v]
__global__ __launch_bounds__(256) void fold_qkv_kernel(const bf16_t* __restrict__ wq, const bf16_t* __restrict__ wk,
                                                       const bf16_t* __restrict__ wv, int n_q_rows, int n_kv_rows,
                                                       int K, const float* __restrict__ gain, int64_t n_units,
                                                       bf16_t* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n_units) return;
  const int upr = K / 8;
  const int r = (int)(u / upr), c = (int)(u % upr) * 8;
  const bf16_t* src = r < n_q_rows ? wq + (int64_t)r * K
                      : r < n_q_rows + n_kv_rows ? wk + (int64_t)(r - n_q_rows) * K
                                                 : wv + (int64_t)(r - n_q_rows - n_kv_rows) * K;
  float v[8], gg[8];
  load8(src + c, v);
  load8(gain + c, gg);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= gg[j];
  store8(out + (int64_t)r * K + c, v);
}

}  // namespace

hipError_t launch_fold_qkv(const void* w_q, const void* w_k, const void* w_v, int n_q_rows, int n_kv_rows, int K,
                           const float* gain, void* out, hipStream_t s) {
  const int64_t n_units = (int64_t)(n_q_rows + 2 * n_kv_rows) * (K / 8);
  if (n_units <= 0) return hipSuccess;
  LaunchScope ls("fold_qkv", s);
  fold_qkv_kernel<<<(unsigned)((n_units + 255) / 256), 256, 0, s>>>((const bf16_t*)w_q, (const bf16_t*)w_k,
                                                                    (const bf16_t*)w_v, n_q_rows, n_kv_rows, K, gain,
                                                                    n_units, (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_pack_gateup(const void* w_gate, const void* w_up, int n_feat, int K, void* packed, hipStream_t s) {
  const int64_t n_chunks = (int64_t)(pack_gateup_bytes(n_feat, K) / 16);
  if (n_chunks == 0) return hipSuccess;
  const int nk = (K + kGateupStep - 1) / kGateupStep;
  LaunchScope ls("pack_gateup", s);
  pack_gateup_kernel<<<(unsigned)((n_chunks + 255) / 256), 256, 0, s>>>((const bf16_t*)w_gate, (const bf16_t*)w_up,
                                                                       n_feat, K, nk, n_chunks, (u32x4_t*)packed);
  return hipGetLastError();
}

hipError_t launch_epilogue_only(const GemmArgs& g0, hipStream_t s) {
  if (g0.M <= 0) return hipSuccess;
  GemmArgs g = g0;
  const int ntiles = gemm_n_tiles(CB_BF16, g.B, g.N);
  const int tpr = (g.epi.kind == EPI_SWIGLU ? BN / 2 : BN) / 8;
  const dim3 rgrid((g.M + 256 / tpr - 1) / (256 / tpr), ntiles);
  LaunchScope ls("epilogue", s);
  switch (g.epi.kind) {
    case EPI_QKV: splitk_epilogue_kernel<EPI_QKV><<<rgrid, 256, 0, s>>>(g, ntiles); break;
    case EPI_RESID: splitk_epilogue_kernel<EPI_RESID><<<rgrid, 256, 0, s>>>(g, ntiles); break;
    default: splitk_epilogue_kernel<EPI_STORE><<<rgrid, 256, 0, s>>>(g, ntiles); break;
  }
  return hipGetLastError();
}

hipError_t launch_resid_norm_only(const GemmArgs& g, const float* gain, float eps, void* hn, hipStream_t s,
                                  bool hn_packed) {
  if (g.M <= 0) return hipSuccess;
  if (hn_packed && g.N % 32) return hipErrorInvalidValue;
  if (g.epi.kind != EPI_RESID || !g.epi.out_f32 || g.N % 8 || g.N > 256 * 8 * kResidNormGroups ||
      g.epi.ld_out != g.N) {
    hipError_t e = launch_epilogue_only(g, s);
    if (e != hipSuccess) return e;
    return launch_rmsnorm(CB_BF16, true, g.epi.out, g.M, nullptr, nullptr, gain, hn, g.M, g.N, eps, s, hn_packed);
  }
  LaunchScope ls("resid_norm", s);
  resid_norm_kernel<<<g.M, 256, 0, s>>>(g, gemm_n_tiles(CB_BF16, g.B, g.N), gain, eps, (bf16_t*)hn, hn_packed);
  return hipGetLastError();
}

int epilogue_ld(int N) { return (N + BN - 1) / BN * BN; }

hipError_t launch_gemm_resid_norm(int dtype, const GemmArgs& g0, const float* gain, float eps, void* hn,
                                  hipStream_t s, bool hn_packed) {
  if (g0.M <= 0) return hipSuccess;
  if (hn_packed && (dtype != CB_BF16 || g0.N % 32)) return hipErrorInvalidValue;
  if (dtype != CB_BF16 || g0.splits <= 1 || g0.epi.kind != EPI_RESID || !g0.epi.out_f32 || g0.N % 8 ||
      g0.N > 256 * 8 * kResidNormGroups || g0.epi.ld_out != g0.N) {
    hipError_t e = launch_gemm(dtype, g0, s);
    if (e != hipSuccess) return e;
    return launch_rmsnorm(dtype, true, g0.epi.out, g0.M, nullptr, nullptr, gain, hn, g0.M, g0.N, eps, s,
                          hn_packed);
  }
  GemmArgs g = g0;
  const int ntiles = gemm_n_tiles(dtype, g.B, g.N);
  const int mt = (g.M + BM - 1) / BM;
  {
    LaunchScope ls("gemm_o", s);
    gemm_bf16_kernel<EPI_RESID, NoShift><<<dim3(mt * ntiles, g.splits), 256, 0, s>>>(g, mt, ntiles, NoShift{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LaunchScope ls("resid_norm", s);
  resid_norm_kernel<<<g.M, 256, 0, s>>>(g, ntiles, gain, eps, (bf16_t*)hn, hn_packed);
  return hipGetLastError();
}

bool gemm_gateup_packed_a(int dtype, int K) {
  return dtype == CB_BF16 && CB_GATEUP_W4 && K % (4 * LBK) == 0;
}

bool gemm_fuses_shift(int dtype, const GemmArgs& g) {
  return dtype == CB_BF16 && g.epi.kind == EPI_QKV && g.B.mode == 0 && g.splits <= 1 && g.epi.req.n == 0 &&
         g.shift && g.shift->kv_dim % 16 == 0;
}

hipError_t launch_gemm(int dtype, const GemmArgs& g0, hipStream_t s) {
  if (g0.M <= 0) return hipSuccess;
  GemmArgs g = g0;
  if (dtype == CB_BF16 && g.B.mode == 1) {
    // gated pair (gate/up): 256-row tiles, no split
    const bool w4 = gemm_gateup_packed_a(dtype, g.K);
    const int tbn = w4 ? kGateupTile : LBN;
    const int nt = (g.B.n_feat + tbn / 2 - 1) / (tbn / 2);
    const int mt = (g.M + LBM - 1) / LBM;
    g.N = nt * tbn;
    g.splits = 1;
    if (g.a_packed && !w4) return hipErrorInvalidValue;
    LaunchScope ls("gemm_gateup", s);
    if (w4)
      gemm_bf16_w4_kernel<EPI_SWIGLU><<<dim3(mt * nt), 256, 0, s>>>(g, mt, nt);
    else
      gemm_bf16_big_kernel<EPI_SWIGLU><<<dim3(mt * nt), kLNT, 0, s>>>(g, mt, nt);
    return hipGetLastError();
  }
  const int ntiles = gemm_n_tiles(dtype, g.B, g.N);
  if (g.B.mode == 1) g.N = ntiles * gemm_bn(dtype);
  if (dtype == CB_BF16) {
    const int mt = (g.M + BM - 1) / BM;
    const dim3 grid(mt * ntiles, g.splits);
    const char* name = g.epi.kind == EPI_QKV ? "gemm_qkv" : g.epi.kind == EPI_SWIGLU ? "gemm_gateup"
                       : g.epi.kind == EPI_RESID && g.epi.out_f32 ? "gemm_o" : "gemm_down";
    if (g.shift && gemm_fuses_shift(dtype, g)) {
      // the layer's re-alignment on the CUs the projection's tiles leave idle
      // (at least 32 workgroups, a multiple of 8 so the tiles keep their XCDs)
      ShiftFuse sf = *g.shift;
      const int tiles = mt * ntiles;
      sf.n_wg = std::max(32, (256 - tiles % 256) / 8 * 8);
      LaunchScope ls(name, s);
      gemm_bf16_kernel<EPI_QKV, ShiftFuse><<<dim3(sf.n_wg + tiles), 256, 0, s>>>(g, mt, ntiles, sf);
      return hipGetLastError();
    }
    {
      LaunchScope ls(name, s);
      switch (g.epi.kind) {
        case EPI_QKV: gemm_bf16_kernel<EPI_QKV, NoShift><<<grid, 256, 0, s>>>(g, mt, ntiles, NoShift{}); break;
        case EPI_RESID: gemm_bf16_kernel<EPI_RESID, NoShift><<<grid, 256, 0, s>>>(g, mt, ntiles, NoShift{}); break;
        case EPI_SWIGLU: gemm_bf16_kernel<EPI_SWIGLU, NoShift><<<grid, 256, 0, s>>>(g, mt, ntiles, NoShift{}); break;
        default: gemm_bf16_kernel<EPI_STORE, NoShift><<<grid, 256, 0, s>>>(g, mt, ntiles, NoShift{}); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits <= 1) return e;
    const int tpr = (g.epi.kind == EPI_SWIGLU ? BN / 2 : BN) / 8;
    const dim3 rgrid((g.M + 256 / tpr - 1) / (256 / tpr), ntiles);
    LaunchScope ls("splitk_epilogue", s);
    switch (g.epi.kind) {
      case EPI_QKV: splitk_epilogue_kernel<EPI_QKV><<<rgrid, 256, 0, s>>>(g, ntiles); break;
      case EPI_RESID: splitk_epilogue_kernel<EPI_RESID><<<rgrid, 256, 0, s>>>(g, ntiles); break;
      case EPI_SWIGLU: splitk_epilogue_kernel<EPI_SWIGLU><<<rgrid, 256, 0, s>>>(g, ntiles); break;
      default: splitk_epilogue_kernel<EPI_STORE><<<rgrid, 256, 0, s>>>(g, ntiles); break;
    }
    return hipGetLastError();
  }
  const int mt = (g.M + FBM - 1) / FBM;
  g.splits = 1;
  LaunchScope ls("gemm_f32", s);
  gemm_f32_kernel<<<dim3(mt * ntiles), dim3(256), 0, s>>>(g, mt, ntiles);
  return hipGetLastError();
}

}  // namespace cb
