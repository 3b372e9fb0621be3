// Deviation analytics (CacheBlend, arXiv 2405.16444, sections 4.1-4.3 and
// Figures 6-8): diagnostics of the fusor, not steps of it.
//
//  * attention deviation (section 4.1): the L-2 (Frobenius) norm of the
//    difference between two forward attention matrices of the same rows,
//    here ||A_a - A_b||^2 and ||A_b||^2 so the caller can form the relative
//    deviation.  A[i][h][t] = softmax over t <= last_key[i] of
//    q[i,h] . k[t, h / (n_q / n_kv)] / sqrt(hd), 0 past last_key[i].
//    One workgroup per (row, head): a first pass over the keys keeps a
//    running max and sum of exponentials per thread for both matrices
//    (combined across the workgroup in a fixed order), a second pass adds
//    (p_a - p_b)^2 and p_b^2 in fp64.  Scores and exponentials are fp32.
//  * Spearman's rank correlation (section 4.3, Figure 8): average ranks
//    (ties share the mean of the ranks they span; one thread per element
//    counts smaller and equal elements), then Pearson's correlation of the
//    ranks in fp64.
//  * top share (Figure 7): the share of the summed values held by the k
//    largest (one thread per element decides membership by counting larger
//    elements and equal ones at lower index).
// Every reduction runs in a fixed order (one workgroup, strided partial sums
// then a tree), so results do not depend on scheduling.
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kAT = 256;   // threads per workgroup

// fixed-order sum of one double per thread over a 256-thread workgroup
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = kAT / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

template <typename T>
__device__ __forceinline__ float dot_row(const float* q, const T* k, int hd) {
  float s = 0.f;
  for (int e = 0; e < hd; ++e) s += q[e] * Elem<T>::ld(k + e);
  return s;
}

template <typename T>
__global__ __launch_bounds__(kAT) void attn_dev_kernel(const T* __restrict__ qa, const T* __restrict__ ka,
                                                       const T* __restrict__ qb, const T* __restrict__ kb,
                                                       const int* __restrict__ last_key, int n_q, int n_kv, int hd,
                                                       int T_rows, float scale, double* __restrict__ part) {
  __shared__ float sq[2][256];
  __shared__ float redf[4][kAT];
  __shared__ double redd[kAT];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int kvh = h / (n_q / n_kv);
  int L = last_key[i] + 1;
  L = L < 1 ? 1 : (L > T_rows ? T_rows : L);
  for (int e = tid; e < hd; e += kAT) {
    sq[0][e] = Elem<T>::ld(qa + ((int64_t)i * n_q + h) * hd + e);
    sq[1][e] = Elem<T>::ld(qb + ((int64_t)i * n_q + h) * hd + e);
  }
  __syncthreads();
  const int ldk = n_kv * hd;
  // pass 1: running max and sum of exponentials per thread, both matrices
  float m[2] = {-INFINITY, -INFINITY}, s[2] = {0.f, 0.f};
  for (int t = tid; t < L; t += kAT) {
    const float x[2] = {dot_row(sq[0], ka + (int64_t)t * ldk + kvh * hd, hd) * scale,
                        dot_row(sq[1], kb + (int64_t)t * ldk + kvh * hd, hd) * scale};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float mn = fmaxf(m[u], x[u]);
      s[u] = s[u] * expf(m[u] - mn) + expf(x[u] - mn);
      m[u] = mn;
    }
  }
  // combine across threads in a fixed order: global max, then rescaled sums
  redf[0][tid] = m[0];
  redf[1][tid] = m[1];
  __syncthreads();
  for (int st = kAT / 2; st > 0; st >>= 1) {
    if (tid < st) {
      redf[0][tid] = fmaxf(redf[0][tid], redf[0][tid + st]);
      redf[1][tid] = fmaxf(redf[1][tid], redf[1][tid + st]);
    }
    __syncthreads();
  }
  const float M[2] = {redf[0][0], redf[1][0]};
  __syncthreads();
  redf[2][tid] = m[0] == -INFINITY ? 0.f : s[0] * expf(m[0] - M[0]);
  redf[3][tid] = m[1] == -INFINITY ? 0.f : s[1] * expf(m[1] - M[1]);
  __syncthreads();
  for (int st = kAT / 2; st > 0; st >>= 1) {
    if (tid < st) {
      redf[2][tid] += redf[2][tid + st];
      redf[3][tid] += redf[3][tid + st];
    }
    __syncthreads();
  }
  const float inv[2] = {1.0f / redf[2][0], 1.0f / redf[3][0]};
  // pass 2: the probabilities again, squared difference and squared norm
  double d2 = 0.0, n2 = 0.0;
  for (int t = tid; t < L; t += kAT) {
    const float pa = expf(dot_row(sq[0], ka + (int64_t)t * ldk + kvh * hd, hd) * scale - M[0]) * inv[0];
    const float pb = expf(dot_row(sq[1], kb + (int64_t)t * ldk + kvh * hd, hd) * scale - M[1]) * inv[1];
    const double df = (double)pa - (double)pb;
    d2 += df * df;
    n2 += (double)pb * (double)pb;
  }
  const double D2 = block_sum(d2, redd);
  const double N2 = block_sum(n2, redd);
  if (tid == 0) {
    part[((int64_t)i * n_q + h) * 2] = D2;
    part[((int64_t)i * n_q + h) * 2 + 1] = N2;
  }
}

// one workgroup: out[0] = sum of part[2j], out[1] = sum of part[2j+1]
__global__ __launch_bounds__(kAT) void sum_pairs_kernel(const double* __restrict__ part, int n, double* out) {
  __shared__ double red[kAT];
  double a = 0.0, b = 0.0;
  for (int j = threadIdx.x; j < n; j += kAT) {
    a += part[2 * (int64_t)j];
    b += part[2 * (int64_t)j + 1];
  }
  const double A = block_sum(a, red);
  const double B = block_sum(b, red);
  if (threadIdx.x == 0) {
    out[0] = A;
    out[1] = B;
  }
}

// average 1-based ranks: smaller + (equal + 1) / 2
__global__ __launch_bounds__(kAT) void rank_kernel(const float* __restrict__ x, int n, double* __restrict__ r) {
  const int i = blockIdx.x * kAT + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  int less = 0, eq = 0;
  for (int j = 0; j < n; ++j) {
    const float w = x[j];
    less += w < v;
    eq += w == v;
  }
  r[i] = (double)less + ((double)eq + 1.0) / 2.0;
}

// one workgroup: Pearson's correlation of rx and ry
__global__ __launch_bounds__(kAT) void pearson_kernel(const double* __restrict__ rx, const double* __restrict__ ry,
                                                      int n, double* out) {
  __shared__ double red[kAT];
  double sx = 0.0, sy = 0.0;
  for (int j = threadIdx.x; j < n; j += kAT) {
    sx += rx[j];
    sy += ry[j];
  }
  const double mx = block_sum(sx, red) / n, my = block_sum(sy, red) / n;
  double xy = 0.0, xx = 0.0, yy = 0.0;
  for (int j = threadIdx.x; j < n; j += kAT) {
    const double a = rx[j] - mx, b = ry[j] - my;
    xy += a * b;
    xx += a * a;
    yy += b * b;
  }
  const double XY = block_sum(xy, red), XX = block_sum(xx, red), YY = block_sum(yy, red);
  if (threadIdx.x == 0) {
    const double den = sqrt(XX * YY);
    out[0] = den > 0.0 ? XY / den : __builtin_nan("");
  }
}

// contribution of element i to the top-k sum: x_i if fewer than k elements
// rank before it (larger, or equal at a lower index), else 0
__global__ __launch_bounds__(kAT) void top_member_kernel(const float* __restrict__ x, int n, int k,
                                                         double* __restrict__ c) {
  const int i = blockIdx.x * kAT + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  int before = 0;
  for (int j = 0; j < n; ++j) {
    const float w = x[j];
    before += (w > v) || (w == v && j < i);
  }
  c[i] = before < k ? (double)v : 0.0;
}

// one workgroup: out[0] = sum(c) / sum(x) (NaN when sum(x) <= 0)
__global__ __launch_bounds__(kAT) void top_share_kernel(const float* __restrict__ x, const double* __restrict__ c,
                                                        int n, double* out) {
  __shared__ double red[kAT];
  double a = 0.0, b = 0.0;
  for (int j = threadIdx.x; j < n; j += kAT) {
    a += c[j];
    b += (double)x[j];
  }
  const double A = block_sum(a, red), B = block_sum(b, red);
  if (threadIdx.x == 0) out[0] = B > 0.0 ? A / B : __builtin_nan("");
}

}  // namespace

hipError_t launch_attention_deviation(int dtype, int m, int n_q, int n_kv, int hd, const void* qa, const void* ka,
                                      const void* qb, const void* kb, int T, const int* last_key, double* part,
                                      double* out, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  const float scale = (float)(1.0 / __builtin_sqrt((double)hd));
  {
    LaunchScope ls("attn_deviation", s);
    const dim3 grid(m, n_q);
    if (dtype == CB_BF16)
      attn_dev_kernel<bf16_t><<<grid, kAT, 0, s>>>((const bf16_t*)qa, (const bf16_t*)ka, (const bf16_t*)qb,
                                                   (const bf16_t*)kb, last_key, n_q, n_kv, hd, T, scale, part);
    else
      attn_dev_kernel<float><<<grid, kAT, 0, s>>>((const float*)qa, (const float*)ka, (const float*)qb,
                                                  (const float*)kb, last_key, n_q, n_kv, hd, T, scale, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LaunchScope ls("attn_deviation_sum", s);
  sum_pairs_kernel<<<1, kAT, 0, s>>>(part, m * n_q, out);
  return hipGetLastError();
}

hipError_t launch_spearman(const float* x, const float* y, int n, double* ranks, double* out, hipStream_t s) {
  LaunchScope ls("spearman", s);
  const unsigned blocks = (unsigned)((n + kAT - 1) / kAT);
  rank_kernel<<<blocks, kAT, 0, s>>>(x, n, ranks);
  rank_kernel<<<blocks, kAT, 0, s>>>(y, n, ranks + n);
  pearson_kernel<<<1, kAT, 0, s>>>(ranks, ranks + n, n, out);
  return hipGetLastError();
}

hipError_t launch_top_share(const float* x, int n, int k, double* contrib, double* out, hipStream_t s) {
  LaunchScope ls("top_share", s);
  top_member_kernel<<<(unsigned)((n + kAT - 1) / kAT), kAT, 0, s>>>(x, n, k, contrib);
  top_share_kernel<<<1, kAT, 0, s>>>(x, contrib, n, out);
  return hipGetLastError();
}

}  // namespace cb
