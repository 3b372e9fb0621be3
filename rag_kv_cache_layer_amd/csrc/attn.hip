// Attention of the recomputed rows over the blended cache.
//
// CacheBlend (arXiv 2405.16444) section 4.2, Figure 5b: the K/V of the
// selected tokens are expanded with the reused entries of all other tokens, so
// that attention includes the selected tokens x all other tokens, and the
// same attention module produces the next layer's input.  Query row i (at
// cache row / position p_i) attends causally to cache rows 0 .. p_i; query
// head h reads KV head h / (n_q / n_kv).
//
// bf16 path (gfx950 matrix cores): one workgroup per (16 query rows, KV head)
// with one wave per query head of the group, so the K/V tiles staged in LDS
// are shared by all heads that read them.  Each wave keeps its 16 queries'
// Q fragments in registers and walks 64-key tiles with an online softmax in
// fp32 (base-2 exponent).  Scores are formed transposed, S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16), so every lane owns one query column: the
// row statistics need only two cross-lane steps and the probabilities feed
// the P V product (O^T += V^T P^T) straight from registers -- the K index of
// an MFMA is a sum, so the same key permutation on both operands is exact.
// V is stored transposed in LDS for that product.  A key tile past a query's
// position is an exact no-op for it (alpha = 1, p = 0), so a row's result
// does not depend on the other rows of its tile.  Tiles holding the latest
// positions (the longest key ranges) are launched first.
//
// fp32 path: one wave per (row, head); scores in LDS, two-pass softmax.
#include "cb_internal.h"

namespace cb {

namespace {

template <int HD, int G>
__global__ __launch_bounds__(64 * G) void attn_bf16_kernel(AttnArgs a, float scale_log2) {
  constexpr int NT = 64 * G;
  constexpr int KT = 64;
  constexpr int KLD = HD + 8;
  constexpr int VLD = KT + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[HD * VLD];
  const int n_tiles = (a.m + 15) / 16;
  const int tile = n_tiles - 1 - (int)blockIdx.x;
  const int kvh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = kvh * G + w;
  const int q = lane & 15, gp = lane >> 4;
  const int i = tile * 16 + q;
  const bool valid = i < a.m;
  int p = valid ? (a.qpos ? a.qpos[i] : i) : 0;
  p = p < 0 ? 0 : (p >= a.T ? a.T - 1 : p);
  int pm = p;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) pm = max(pm, __shfl_xor(pm, o));

  const int ldq = a.n_q * HD, ldkv = a.n_kv * HD;
  bf16x8_t qf[HD / 32];
  {
    const int qr = valid ? (a.qmap ? a.qmap[i] : i) : 0;
    const bf16_t* Qp = (const bf16_t*)a.Q + (int64_t)qr * ldq + head * HD + gp * 8;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
      uint4 u = valid ? *reinterpret_cast<const uint4*>(Qp + ks * 32) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  f32x4_t oacc[HD / 16];
#pragma unroll
  for (int mb = 0; mb < HD / 16; ++mb) oacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const bf16_t* Kg = (const bf16_t*)a.K + kvh * HD;
  const bf16_t* Vg = (const bf16_t*)a.V + kvh * HD;

  for (int t0 = 0; t0 <= pm; t0 += KT) {
    for (int c = tid; c < KT * HD / 8; c += NT) {
      const int r = c / (HD / 8), cc = (c % (HD / 8)) * 8;
      const int t = t0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (t < a.T) {
        kv = *reinterpret_cast<const uint4*>(Kg + (int64_t)t * ldkv + cc);
        vv = *reinterpret_cast<const uint4*>(Vg + (int64_t)t * ldkv + cc);
      }
      *reinterpret_cast<uint4*>(Ks + r * KLD + cc) = kv;
      const uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Vt[(cc + 2 * j) * VLD + r] = (bf16_t)(wv[j] & 0xffffu);
        Vt[(cc + 2 * j + 1) * VLD + r] = (bf16_t)(wv[j] >> 16);
      }
    }
    __syncthreads();

    // S^T[key][query] for 4 blocks of 16 keys; lane holds keys 16kb+4gp+v of query q
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Ks + (kb * 16 + q) * KLD + ks * 32 + gp * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = t0 + kb * 16 + 4 * gp + v;
        const float x = key <= p ? s[kb][v] * scale_log2 : -INFINITY;
        s[kb][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = exp2f(s[kb][v] - m_new);
        s[kb][v] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < HD / 16; ++mb) oacc[mb] *= alpha;

    // P^T as the B operand: k slot j of lane group gp is key 32st+4gp+j (j<4)
    // or 32st+16+4gp+(j-4) (j>=4), matching the A operand read from V^T below.
    bf16x8_t pb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pb[st][v] = (__bf16)s[2 * st][v];
        pb[st][4 + v] = (__bf16)s[2 * st + 1][v];
      }
#pragma unroll
    for (int mb = 0; mb < HD / 16; ++mb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16_t* vr = Vt + (mb * 16 + q) * VLD + st * 32 + 4 * gp;
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vr);
        const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(vr + 16);
        const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[st], oacc[mb], 0, 0, 0);
      }
    __syncthreads();
  }

  if (valid) {
    const float inv = 1.0f / l_run;
    bf16_t* Op = (bf16_t*)a.O + (int64_t)i * ldq + head * HD + 4 * gp;
#pragma unroll
    for (int mb = 0; mb < HD / 16; ++mb) {
      const uint32_t w0 = (uint32_t)f2bf(oacc[mb][0] * inv) | ((uint32_t)f2bf(oacc[mb][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f2bf(oacc[mb][2] * inv) | ((uint32_t)f2bf(oacc[mb][3] * inv) << 16);
      *reinterpret_cast<uint2*>(Op + mb * 16) = make_uint2(w0, w1);
    }
  }
}

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, float scale) {
  extern __shared__ float sc[];
  __shared__ float qs[256];
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int hd = a.hd;
  const int kvh = h / (a.n_q / a.n_kv);
  int p = a.qpos ? a.qpos[i] : i;
  p = p < 0 ? 0 : (p >= a.T ? a.T - 1 : p);
  const int qr = a.qmap ? a.qmap[i] : i;
  const float* Qp = (const float*)a.Q + (int64_t)qr * a.n_q * hd + h * hd;
  for (int d = lane; d < hd; d += 64) qs[d] = Qp[d];
  __syncthreads();
  const int ldkv = a.n_kv * hd;
  const float* Kg = (const float*)a.K + kvh * hd;
  const float* Vg = (const float*)a.V + kvh * hd;
  float mx = -INFINITY;
  for (int t = lane; t <= p; t += 64) {
    const float* kr = Kg + (int64_t)t * ldkv;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += qs[d] * kr[d];
    s *= scale;
    sc[t] = s;
    mx = fmaxf(mx, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float sum = 0.f;
  for (int t = lane; t <= p; t += 64) {
    const float e = expf(sc[t] - mx);
    sc[t] = e;
    sum += e;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  __syncthreads();
  float* Op = (float*)a.O + (int64_t)i * a.n_q * hd + h * hd;
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    for (int t = 0; t <= p; ++t) acc += sc[t] * Vg[(int64_t)t * ldkv + d];
    Op[d] = acc / sum;
  }
}

template <int HD>
hipError_t launch_bf16_hd(const AttnArgs& a, hipStream_t s, float scale_log2) {
  const int g = a.n_q / a.n_kv;
  const dim3 grid((a.m + 15) / 16, a.n_kv);
  switch (g) {
    case 1: attn_bf16_kernel<HD, 1><<<grid, 64, 0, s>>>(a, scale_log2); break;
    case 2: attn_bf16_kernel<HD, 2><<<grid, 128, 0, s>>>(a, scale_log2); break;
    case 4: attn_bf16_kernel<HD, 4><<<grid, 256, 0, s>>>(a, scale_log2); break;
    case 8: attn_bf16_kernel<HD, 8><<<grid, 512, 0, s>>>(a, scale_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.m <= 0) return hipSuccess;
  LaunchScope ls("attention", s);
  if (dtype == CB_BF16) {
    const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.hd));
    if (a.hd == 128) return launch_bf16_hd<128>(a, s, scale_log2);
    if (a.hd == 64) return launch_bf16_hd<64>(a, s, scale_log2);
    return hipErrorInvalidValue;
  }
  const float scale = (float)(1.0 / __builtin_sqrt((double)a.hd));
  attn_f32_kernel<<<dim3(a.m, a.n_q), 64, (size_t)a.T * sizeof(float), s>>>(a, scale);
  return hipGetLastError();
}

}  // namespace cb
