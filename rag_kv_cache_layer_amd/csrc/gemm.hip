// Projections of the recomputed rows: C[M][N] = A[M][K] * B[N][K]^T.
//
// CacheBlend (arXiv 2405.16444) section 4.2, Figure 5b: only the selected
// tokens' rows go through the layer's projections, so these are dense
// contractions with a small M (the selected rows) against the full weight
// matrices -- the part of the fusor that really is GEMM-shaped.  B is the
// nn.Linear weight [out][in], so both operands are contiguous along K.
//
// bf16 path (gfx950 matrix cores): 256 threads, 128x128 output tile, K step
// 64, four waves of 64x64, each a 4x4 grid of v_mfma_f32_16x16x32_bf16.
// Operands are staged through double-buffered LDS (rows padded by 16 B so the
// 16-byte fragment reads of 16 rows hit distinct banks).  Tiles are numbered
// so that the M tiles sharing one weight tile run back to back on the same
// XCD (workgroups are dealt round-robin to the 8 XCDs), which keeps each
// weight tile in that XCD's L2 while it is reused.  Split-K (chosen from N
// and K only, never from M) writes fp32 partials that a second kernel sums in
// a fixed order, so a row's result never depends on how many rows there are.
//
// fp32 path: a 64x64 SIMT tile kernel (exact fp32 products, fp32 accumulate)
// for the fp32 configuration.
//
// Epilogues (applied from an fp32 tile in LDS, 8 consecutive columns per
// thread): QKV (RoPE at each row's absolute position on Q and K, per-row K
// deviation against the cached row before it is replaced, scatter of K/V into
// the cache), residual add, and SwiGLU on interleaved gate/up tiles.
#include "cb_internal.h"

namespace cb {

namespace {

// bf16 tiles
constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8, CLD = BN + 4;
constexpr int kGemmSmem = 2 * (BM + BN) * LDK * 2;  // 73728 B
static_assert(BM * CLD * 4 <= kGemmSmem, "C tile must fit in the operand buffers");
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
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = v[2 * j], b = v[2 * j + 1];
    v[2 * j] = a * cs[j] - b * sn[j];
    v[2 * j + 1] = a * sn[j] + b * cs[j];
  }
}

// Q/K/V columns: returns this group's contribution to the row's K deviation.
template <typename T>
__device__ float epi_qkv(const EpiParams& e, int gm, int c, float v[8]) {
  const int crow = e.rows ? e.rows[gm] : gm;
  if (crow < 0 || crow >= e.T) return 0.f;
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
    T* kp = (T*)e.k_cache + (int64_t)crow * e.kv_dim + (c - e.q_dim);
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = Elem<T>::rnd(v[j]);
    float contrib = 0.f;
    if (e.dev_part && crow >= e.dev_lo && crow < e.dev_hi) {
      float old[8];
      load8(kp, old);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = r[j] - old[j];
        contrib += d * d;
      }
    }
    store8(kp, r);
    return contrib;
  }
  store8((T*)e.v_cache + (int64_t)crow * e.kv_dim + (c - e.q_dim - e.kv_dim), v);
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
  for (int j = 0; j < 8; ++j) o[j] = (g[j] / (1.0f + expf(-g[j]))) * u[j];
  store8((T*)e.out + (int64_t)gm * e.ld_out + f, o);
}

template <typename T>
__device__ void epi_store(const EpiParams& e, int gm, int c, const float v[8]) {
  if (e.out_f32) store8((float*)e.out + (int64_t)gm * e.ld_out + c, v);
  else store8((T*)e.out + (int64_t)gm * e.ld_out + c, v);
}

// Apply the epilogue to a bm x bn fp32 tile held in LDS (row stride cld).
template <typename T, int bm, int bn, int NT>
__device__ void run_epilogue(const EpiParams& e, const BOperand& B, const float* Cs, int cld, int m0, int tn,
                             int M, int N) {
  const bool swiglu = e.kind == EPI_SWIGLU;
  const int cols = swiglu ? bn / 2 : bn;
  const int tpr = cols / 8;  // threads per row (power of two, <= 64)
  const int rpp = NT / tpr;
  const int tid = threadIdx.x;
  const int lr = tid / tpr, lc = (tid % tpr) * 8;
  const bool want_dev = e.kind == EPI_QKV && e.dev_part != nullptr;
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
      if (swiglu) {
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
          if (e.kind == EPI_QKV) contrib = epi_qkv<T>(e, gm, c, v);
          else if (e.kind == EPI_RESID) epi_resid<T>(e, gm, c, v);
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

__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs g, int mt, int ntiles) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmSmem];
  bf16_t* As = (bf16_t*)smem;            // [2][BM][LDK]
  bf16_t* Bs = As + 2 * BM * LDK;        // [2][BN][LDK]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * BM;
  const int M = g.M, K = g.K;
  const int kchunk = ((K + g.splits - 1) / g.splits + BK - 1) / BK * BK;
  const int kb = blockIdx.y * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  // Loader: each thread moves 4 A and 4 B chunks of 16 B per K step.  The
  // addresses are always in bounds (invalid rows fall back to row 0 / the
  // weight's first row, the K tail to the first chunk of this split) and the
  // zero fill is applied when the chunk is written to LDS, so no loaded value
  // is consumed before the MFMAs of the current step have been issued.
  typedef __attribute__((address_space(1))) const u32x4_t guint4;
  const guint4* ag[4];
  const guint4* bg[4];
  bool aok[4], bok[4];
  int lrow[4], lcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    lrow[i] = c >> 3;
    lcol[i] = (c & 7) * 8;
    aok[i] = m0 + lrow[i] < M;
    ag[i] = (const guint4*)((const bf16_t*)g.A + (int64_t)(aok[i] ? m0 + lrow[i] : 0) * K);
    const bf16_t* br = b_row<bf16_t>(g.B, K, g.N, tn, BN, lrow[i]);
    bok[i] = br != nullptr;
    bg[i] = (const guint4*)(bok[i] ? br : (const bf16_t*)g.B.p0);
  }
  u32x4_t ra[4], rb[4];
  const u32x4_t z4 = {0u, 0u, 0u, 0u};

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = kb + lcol[i];
      const int kc = (kk < ke ? kk : kb) >> 3;
      ra[i] = ag[i][kc];
      rb[i] = bg[i][kc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool kin = kb + lcol[i] < ke;
      *reinterpret_cast<u32x4_t*>(As + lrow[i] * LDK + lcol[i]) = (aok[i] && kin) ? ra[i] : z4;
      *reinterpret_cast<u32x4_t*>(Bs + lrow[i] * LDK + lcol[i]) = (bok[i] && kin) ? rb[i] : z4;
    }
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const int kn = kb + (it + 1) * BK;  // next K step
    const bool more = it + 1 < nk;
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kn + lcol[i];
        const int kc = (kk < ke ? kk : kb) >> 3;
        ra[i] = ag[i][kc];
        rb[i] = bg[i][kc];
      }
    }
    const bf16_t* Ac = As + cur * BM * LDK;
    const bf16_t* Bc = Bs + cur * BN * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(Ac + (wm + i * 16 + fr) * LDK + ks * 32 + fk);
        bfr[i] = *reinterpret_cast<const bf16x8_t*>(Bc + (wn + i * 16 + fr) * LDK + ks * 32 + fk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16_t* An = As + (cur ^ 1) * BM * LDK;
      bf16_t* Bn = Bs + (cur ^ 1) * BN * LDK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool kin = kn + lcol[i] < ke;
        *reinterpret_cast<u32x4_t*>(An + lrow[i] * LDK + lcol[i]) = (aok[i] && kin) ? ra[i] : z4;
        *reinterpret_cast<u32x4_t*>(Bn + lrow[i] * LDK + lcol[i]) = (bok[i] && kin) ? rb[i] : z4;
      }
    }
    __syncthreads();
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
        Cs[(wm + i * 16 + (lane >> 4) * 4 + v) * CLD + wn + j * 16 + fr] = acc[i][j][v];
  __syncthreads();

  if (g.splits > 1) {
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
  run_epilogue<bf16_t, BM, BN, 256>(g.epi, g.B, Cs, CLD, m0, tn, M, g.N);
}

// Sum the split-K partials of one tile in split order, then run the epilogue.
template <typename T, int bm, int bn>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int mt, int ntiles) {
  __shared__ __attribute__((aligned(16))) float Cs[bm * (bn + 4)];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x % mt, tn = blockIdx.x / mt;
  const int m0 = tm * bm, M = g.M;
  const int ldp = ntiles * bn;
  for (int idx = tid; idx < bm * bn / 4; idx += 256) {
    const int r = idx / (bn / 4), c4 = (idx % (bn / 4)) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m0 + r < M) {
      for (int sp = 0; sp < g.splits; ++sp) {
        const float4 p =
            *reinterpret_cast<const float4*>(g.part + ((int64_t)sp * M + m0 + r) * ldp + tn * bn + c4);
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
      }
    }
    *reinterpret_cast<float4*>(Cs + r * (bn + 4) + c4) = s;
  }
  __syncthreads();
  run_epilogue<T, bm, bn, 256>(g.epi, g.B, Cs, bn + 4, m0, tn, M, g.N);
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
  run_epilogue<float, FBM, FBN, 256>(g.epi, g.B, Cs, FCLD, m0, tn, M, g.N);
}

}  // namespace

int gemm_bn(int dtype) { return dtype == CB_BF16 ? BN : FBN; }

int gemm_n_tiles(int dtype, const BOperand& B, int N) {
  const int bn = gemm_bn(dtype);
  if (B.mode == 1) return (B.n_feat + bn / 2 - 1) / (bn / 2);
  return (N + bn - 1) / bn;
}

int gemm_splits(int dtype, int n_tiles, int K) {
  if (dtype != CB_BF16) return 1;
  int s = 1;
  while (s < 4 && n_tiles * s < 64 && K / (2 * s) >= 1024) s *= 2;
  return s;
}

hipError_t launch_gemm(int dtype, const GemmArgs& g0, hipStream_t s) {
  if (g0.M <= 0) return hipSuccess;
  GemmArgs g = g0;
  const int ntiles = gemm_n_tiles(dtype, g.B, g.N);
  if (g.B.mode == 1) g.N = ntiles * gemm_bn(dtype);
  if (dtype == CB_BF16) {
    const int mt = (g.M + BM - 1) / BM;
    {
      LaunchScope ls(g.epi.kind == EPI_QKV ? "gemm_qkv" : g.epi.kind == EPI_SWIGLU ? "gemm_gateup"
                     : g.epi.kind == EPI_RESID && g.epi.out_f32 ? "gemm_o" : "gemm_down", s);
      gemm_bf16_kernel<<<dim3(mt * ntiles, g.splits), dim3(256), 0, s>>>(g, mt, ntiles);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits <= 1) return e;
    LaunchScope ls("splitk_reduce", s);
    splitk_reduce_kernel<bf16_t, BM, BN><<<dim3(mt * ntiles), dim3(256), 0, s>>>(g, mt, ntiles);
    return hipGetLastError();
  }
  const int mt = (g.M + FBM - 1) / FBM;
  g.splits = 1;
  LaunchScope ls("gemm_f32", s);
  gemm_f32_kernel<<<dim3(mt * ntiles), dim3(256), 0, s>>>(g, mt, ntiles);
  return hipGetLastError();
}

}  // namespace cb
