// 8-bit float operands for the projections (the paper serves its larger
// models with 8-bit weights, CacheBlend section 7): OCP fp8 E4M3 with one
// power-of-two scale per matrix row.
//
// quantize_rows_kernel: one workgroup per row.  e = the smallest integer with
// amax <= 448 * 2^e, found from the bits of amax (amax = m * 2^E, m in [1,2):
// e = E - 8 + (m > 1.75)); every element is scaled by 2^-e (exact), clamped
// to +-448 and rounded to the nearest E4M3 value, ties to even
// (v_cvt_pk_fp8_f32).
//
// gemm_fp8_kernel: C = (A B^T) * 2^(e_a[row] + e_b[col]) for fp8 A [M][K] and
// B [N][K].  128x128 tiles, 4 waves of 64x64 built from
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit block scales; every
// product is exact in fp32).  K steps of 128 bytes: a row step is 128 bytes
// as in the bf16 kernel's 64-element steps, so the same direct-to-LDS ring
// and XOR swizzle serve, and each MFMA takes two adjacent 16-byte chunks of
// a row.  The K index of an MFMA is a sum, so any assignment of a row's 128
// bytes to lanes that A and B share gives the same product.  Split-K
// partials are scaled before they are written (exact) and summed in split
// order.
#include "cb_internal.h"

namespace cb {

namespace {

#ifndef CB_FP8_NSTAGE
#define CB_FP8_NSTAGE 3
#endif
constexpr int QBM = 128, QBN = 128, QBK = 128, QNS = CB_FP8_NSTAGE, QCLD = QBN + 4;
constexpr int kQStage = (QBM + QBN) * QBK;                   // 32 KB
constexpr int kQSmem = QNS * kQStage > QBM * QCLD * 4 ? QNS * kQStage : QBM * QCLD * 4;
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int qswz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = 2.f * frexpf(amax, &E);   // amax = m * 2^(E-1), m in [1, 2)
  return (E - 1) - 8 + (m > 1.75f ? 1 : 0);
}

// one workgroup per row; with vec (rows a multiple of 16 elements, 16-byte
// aligned buffers) each thread takes 16 consecutive elements per pass (16-byte
// loads, one 16-byte store of codes), otherwise element by element
template <typename T>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ x, int cols, bool vec,
                                                            uint8_t* __restrict__ q, int* __restrict__ ex) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const T* xr = x + (int64_t)row * cols;
  uint8_t* qr = q + (int64_t)row * cols;
  const int vec_end = vec ? cols : 0;
  float amax = 0.f;
  for (int c = tid * 16; c < vec_end; c += 256 * 16) {
    float v[16];
    load8(xr + c, v);
    load8(xr + c + 8, v + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  for (int c = vec_end + tid; c < cols; c += 256) amax = fmaxf(amax, fabsf(Elem<T>::ld(xr + c)));
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = row_exponent(amax);
  if (tid == 0) ex[row] = e;
  auto scaled = [&](float v) { return fminf(fmaxf(ldexpf(v, -e), -448.f), 448.f); };
  for (int c = tid * 16; c < vec_end; c += 256 * 16) {
    float v[16];
    load8(xr + c, v);
    load8(xr + c + 8, v + 8);
    u32x4_t w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(v[4 * j]), scaled(v[4 * j + 1]), 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(v[4 * j + 2]), scaled(v[4 * j + 3]), pk, true);
      w[j] = (uint32_t)pk;
    }
    *reinterpret_cast<u32x4_t*>(qr + c) = w;
  }
  for (int c = vec_end + tid; c < cols; c += 256)
    qr[c] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(scaled(Elem<T>::ld(xr + c)), 0.f, 0, false) & 0xff);
}

template <typename TO>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(Fp8GemmArgs g, int mt, int ntiles) {
  __shared__ __attribute__((aligned(16))) char smem[kQSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = (gridDim.x & 7) == 0 ? ((int)blockIdx.x & 7) * (gridDim.x >> 3) + ((int)blockIdx.x >> 3)
                                      : (int)blockIdx.x;
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * QBM, n0 = tn * QBN;
  const int M = g.M, N = g.N, K = g.K;
  const int kchunk = ((K + g.splits - 1) / g.splits + QBK - 1) / QBK * QBK;
  const int kb = blockIdx.y * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nk = ke > kb ? (ke - kb + QBK - 1) / QBK : 0;

  // DMA plan (as the bf16 128x128 kernel): wave w fills row groups
  // (w*4 + j)*8 .. +7 of the A and B tiles; lane i fills slot i%8 of row i/8
  // with the logical chunk slot ^ ((row >> 1) & 7); out-of-range rows and K
  // past ke load as zero.
  const uint32_t kOOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)M * K));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)N * K));
  uint32_t aoff[4], boff[4];
  int lcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (w * 4 + j) * 8 + (lane >> 3);
    lcol[j] = ((lane & 7) ^ ((row >> 1) & 7)) * 16;
    aoff[j] = m0 + row < M ? (uint32_t)((int64_t)(m0 + row) * K) : kOOB;
    boff[j] = n0 + row < N ? (uint32_t)((int64_t)(n0 + row) * K) : kOOB;
  }
  // row group j of the A and B tiles of one stage (two wave instructions)
  auto issue_group = [&](int stage, int k0, int j) {
    char* sa = smem + stage * kQStage;
    char* sb = sa + QBM * QBK;
    const int grp = w * 4 + j;
    const int kk = k0 + lcol[j];
    const bool kin = kk < ke;
    const uint32_t oa = (kin && aoff[j] != kOOB) ? aoff[j] + kk : kOOB;
    const uint32_t ob = (kin && boff[j] != kOOB) ? boff[j] + kk : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + grp * 1024), 16, oa, 0, 0, CB_A_AUX);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sb + grp * 1024), 16, ob, 0, 0, CB_W_AUX);
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
  const int fr = lane & 15, fc = lane >> 4;   // lane group fc takes chunks 2fc, 2fc+1 of the row
  auto frag = [&](const char* base, int r) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + qswz(r, 2 * fc));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + qswz(r, 2 * fc + 1));
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto compute = [&](int stage) {
    const char* sa = smem + stage * kQStage;
    const char* sb = sa + QBM * QBK;
    i32x8_t af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = frag(sa, wm + i * 16 + fr);
      bfr[i] = frag(sb, wn + i * 16 + fr);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0,
                                                                      127);
    }
  };

#pragma unroll
  for (int st = 0; st < QNS - 1; ++st)
    if (st < nk) issue(st, kb + st * QBK);
  for (int it0 = 0; it0 < nk; it0 += QNS) {
#pragma unroll
    for (int u = 0; u < QNS; ++u) {
      const int it = it0 + u;
      if (it < nk) {
        // this wave's loads of step it landed once at most the later steps'
        // (8 loads each, only those actually issued) are outstanding
        const int later = min(nk - 1 - it, QNS - 2);
        static_assert(QNS >= 2 && QNS <= 5, "wait counts below cover at most three later steps");
        if (later >= 3) CB_WAIT_VMCNT(24);
        else if (later == 2) CB_WAIT_VMCNT(16);
        else if (later == 1) CB_WAIT_VMCNT(8);
        else CB_WAIT_VMCNT(0);
        CB_BARRIER();
        if (it + QNS - 1 < nk) issue((u + QNS - 1) % QNS, kb + (it + QNS - 1) * QBK);
        compute(u);
      }
    }
  }
  CB_WAIT_VMCNT(0);
  __syncthreads();

  // scale by 2^(e_a + e_b) (exact) and write through an fp32 tile in LDS
  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 16 + fr;
      const int eb = col < N ? g.b_exp[col] : 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm + i * 16 + fc * 4 + v;
        const int ea = row < M ? g.a_exp[row] : 0;
        Cs[(wm + i * 16 + fc * 4 + v) * QCLD + wn + j * 16 + fr] = ldexpf(acc[i][j][v], ea + eb);
      }
    }
  __syncthreads();
  if (g.splits > 1) {
    float* P = g.part + (int64_t)blockIdx.y * M * N;
    for (int idx = tid; idx < QBM * QBN; idx += 256) {
      const int r = idx / QBN, c = idx % QBN;
      if (m0 + r < M && n0 + c < N) P[(int64_t)(m0 + r) * N + n0 + c] = Cs[r * QCLD + c];
    }
    return;
  }
  for (int idx = tid; idx < QBM * QBN; idx += 256) {
    const int r = idx / QBN, c = idx % QBN;
    if (m0 + r < M && n0 + c < N) Elem<TO>::st((TO*)g.C + (int64_t)(m0 + r) * g.ldc + n0 + c, Cs[r * QCLD + c]);
  }
}

// gemm_fp8_big_kernel: the same product on 256x256 tiles for wide outputs
// (enough tiles to fill the chip without split-K).  Gated mode (gate/up of a
// SwiGLU MLP, B = [W_gate; W_up]): tile tn holds gate rows 128 tn .. +127 in
// its first 128 columns and the same up rows in the last 128, and the
// epilogue writes silu(gate) * up for those 128 features.  8 waves of 128x64, K
// steps of 128 bytes, a two-stage LDS ring of 64 KB stages filled by
// direct-to-LDS loads (the 128-byte row swizzle of the 128x128 kernel), with
// the next stage's loads issued one 1 KB block per MFMA row.  A 256x256 tile
// moves half the bytes per flop of a 128x128 one, which is what limits these
// kernels.
constexpr int QLM = 256, QLN = 256, QLNS = 2, QLCLD = QLN + 4;
constexpr int kQLStage = (QLM + QLN) * QBK;                                   // 64 KB
constexpr int kQLSmem = QLNS * kQLStage > 128 * QLCLD * 4 ? QLNS * kQLStage : 128 * QLCLD * 4;
constexpr int kQLBlocksA = QLM / 8;                                           // 1 KB blocks of A per stage

template <typename TO>
__global__ __launch_bounds__(512, 1) void gemm_fp8_big_kernel(Fp8GemmArgs g, int mt, int ntiles) {
  __shared__ __attribute__((aligned(16))) char smem[kQLSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = (gridDim.x & 7) == 0 ? ((int)blockIdx.x & 7) * (gridDim.x >> 3) + ((int)blockIdx.x >> 3)
                                      : (int)blockIdx.x;
  const int tm = id % mt, tn = id / mt;
  const int m0 = tm * QLM, n0 = tn * QLN;
  const int M = g.M, N = g.N, K = g.K;
  const int nk = (K + QBK - 1) / QBK;
  const int GF = g.gated_F;
  // weight row of tile column c (-1 past the end)
  auto brow_of = [&](int c) {
    if (GF == 0) return n0 + c < N ? n0 + c : -1;
    const int f = tn * (QLN / 2) + (c % (QLN / 2));
    return f < GF ? (c < QLN / 2 ? f : GF + f) : -1;
  };

  // DMA plan: block b of a stage holds tile rows 8b .. 8b+7 (A's 256 rows,
  // then B's); wave w fills blocks w + 8j; lane i fills slot i % 8 of row
  // i / 8 with the logical chunk slot ^ ((row >> 1) & 7)
  const uint32_t kOOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)M * K));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)N * K));
  uint32_t off[8];
  int lcol[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int blk = w + 8 * j;
    const bool is_a = blk < kQLBlocksA;
    const int row = (is_a ? blk : blk - kQLBlocksA) * 8 + (lane >> 3);
    lcol[j] = ((lane & 7) ^ ((row >> 1) & 7)) * 16;
    const int grow = is_a ? (m0 + row < M ? m0 + row : -1) : brow_of(row);
    off[j] = grow >= 0 ? (uint32_t)((int64_t)grow * K) : kOOB;
  }
  auto issue_group = [&](int stage, int k0, int j) {
    const int blk = w + 8 * j;
    const int kk = k0 + lcol[j];
    const uint32_t o = (kk < K && off[j] != kOOB) ? off[j] + kk : kOOB;
    static_assert(kQLBlocksA % 8 == 0, "block w + 8 j is an activation block exactly when 8 j < kQLBlocksA");
    if (8 * j < kQLBlocksA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(smem + stage * kQLStage + blk * 1024), 16, o, 0, 0,
                                               CB_A_AUX);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(smem + stage * kQLStage + blk * 1024), 16, o, 0, 0,
                                               CB_W_AUX);
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wm = (w >> 2) * 128, wn = (w & 3) * 64;
  const int fr = lane & 15, fc = lane >> 4;
  auto frag = [&](const char* base, int r) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + qswz(r, 2 * fc));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + qswz(r, 2 * fc + 1));
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

#pragma unroll
  for (int j = 0; j < 8; ++j) issue_group(0, 0, j);
  for (int it = 0; it < nk; ++it) {
    CB_WAIT_VMCNT(0);   // this wave's blocks of step it landed (nothing later is in flight)
    CB_BARRIER();       // every wave's, and every wave is done reading the other stage
    const int stage = it & 1;
    const bool more = it + 1 < nk;
    const char* sa = smem + stage * kQLStage;
    const char* sb = sa + QLM * QBK;
    i32x8_t af[8], bfr[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = frag(sa, wm + i * 16 + fr);
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = frag(sb, wn + j * 16 + fr);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0,
                                                                      127);
      if (more) {
        __builtin_amdgcn_sched_barrier(0);
        issue_group(stage ^ 1, (it + 1) * QBK, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  CB_WAIT_VMCNT(0);
  __syncthreads();

  // scale by 2^(e_a + e_b) (exact); write through an fp32 tile of 128 rows
  float* Cs = (float*)smem;
  const bool vec = (g.ldc & 7) == 0 && ((uintptr_t)g.C & 15) == 0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wm >> 7) == half) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int br = brow_of(wn + j * 16 + fr);
          const int eb = br >= 0 ? g.b_exp[br] : 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rr = i * 16 + fc * 4 + v;   // row within the half
            const int row = m0 + half * 128 + rr;
            const int ea = row < M ? g.a_exp[row] : 0;
            Cs[rr * QLCLD + wn + j * 16 + fr] = ldexpf(acc[i][j][v], ea + eb);
          }
        }
    }
    __syncthreads();
    if (GF > 0) {
      // u = silu(gate) * up for features 128 tn .. +127, bf16
      for (int idx = tid; idx < 128 * (QLN / 16); idx += 512) {
        const int r = idx / (QLN / 16), c = (idx % (QLN / 16)) * 8;
        const int row = m0 + half * 128 + r, f = tn * (QLN / 2) + c;
        if (row >= M || f >= GF) continue;
        const float* gp = Cs + r * QLCLD + c;
        float o[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) o[x] = silu(gp[x]) * gp[x + QLN / 2];
        bf16_t* dst = (bf16_t*)g.C + (int64_t)row * g.ldc + f;
        if (vec && f + 8 <= GF) {
          store8(dst, o);
        } else {
          for (int x = 0; x < 8 && f + x < GF; ++x) Elem<bf16_t>::st(dst + x, o[x]);
        }
      }
      __syncthreads();
      continue;
    }
    for (int idx = tid; idx < 128 * (QLN / 8); idx += 512) {
      const int r = idx / (QLN / 8), c = (idx % (QLN / 8)) * 8;
      const int row = m0 + half * 128 + r, col = n0 + c;
      if (row >= M) continue;
      TO* dst = (TO*)g.C + (int64_t)row * g.ldc + col;
      const float* src = Cs + r * QLCLD + c;
      if (vec && col + 8 <= N) {
        store8(dst, src);
      } else {
        for (int x = 0; x < 8 && col + x < N; ++x) Elem<TO>::st(dst + x, src[x]);
      }
    }
    __syncthreads();
  }
}

template <typename TO>
__global__ __launch_bounds__(256) void fp8_split_sum_kernel(Fp8GemmArgs g) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.M * g.N) return;
  float s = 0.f;
  for (int sp = 0; sp < g.splits; ++sp) s += g.part[(int64_t)sp * g.M * g.N + i];
  const int64_t r = i / g.N, c = i % g.N;
  Elem<TO>::st((TO*)g.C + r * g.ldc + c, s);
}

}  // namespace

int fp8_splits(int N, int K) {
  const int nt = (N + QBN - 1) / QBN;
  int s = 1;
  while (s < 4 && nt * s < 48 && K / (2 * s) >= 1024) s *= 2;
  return s;
}

hipError_t launch_quantize_rows(int src_dtype, const void* x, int rows, int cols, uint8_t* q, int* ex,
                                hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  LaunchScope ls("quantize_fp8", s);
  const bool vec = cols % 16 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)q & 15) == 0;
  if (src_dtype == CB_BF16)
    quantize_rows_kernel<bf16_t><<<rows, 256, 0, s>>>((const bf16_t*)x, cols, vec, q, ex);
  else
    quantize_rows_kernel<float><<<rows, 256, 0, s>>>((const float*)x, cols, vec, q, ex);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const Fp8GemmArgs& g, int out_dtype, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  {
    // wide outputs: 256x256 tiles when they alone give ~3/4 of a wave of
    // workgroups per CU (the 128x128 kernel would not split K either)
    const int lmt = (g.M + QLM - 1) / QLM;
    const int lnt = g.gated_F > 0 ? (g.gated_F + QLN / 2 - 1) / (QLN / 2) : (g.N + QLN - 1) / QLN;
    if (g.gated_F > 0 || (g.splits == 1 && lmt * lnt >= 192)) {
      LaunchScope ls(g.gated_F > 0 ? "gemm_fp8_gateup" : "gemm_fp8_big", s);
      if (out_dtype == CB_BF16) gemm_fp8_big_kernel<bf16_t><<<lmt * lnt, 512, 0, s>>>(g, lmt, lnt);
      else gemm_fp8_big_kernel<float><<<lmt * lnt, 512, 0, s>>>(g, lmt, lnt);
      return hipGetLastError();
    }
  }
  const int mt = (g.M + QBM - 1) / QBM, nt = (g.N + QBN - 1) / QBN;
  const dim3 grid(mt * nt, g.splits);
  {
    LaunchScope ls("gemm_fp8", s);
    if (out_dtype == CB_BF16) gemm_fp8_kernel<bf16_t><<<grid, 256, 0, s>>>(g, mt, nt);
    else gemm_fp8_kernel<float><<<grid, 256, 0, s>>>(g, mt, nt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.splits <= 1 || g.keep_parts) return e;
  LaunchScope ls("gemm_fp8_split_sum", s);
  const int64_t n = (int64_t)g.M * g.N;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (out_dtype == CB_BF16) fp8_split_sum_kernel<bf16_t><<<blocks, 256, 0, s>>>(g);
  else fp8_split_sum_kernel<float><<<blocks, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace cb
