// RMSNorm of gathered rows (the layer-input mask of CacheBlend section 4.2,
// Figure 5b, fused with the layer's first normalisation):
//   out[i] = x[map(i)] / sqrt(mean(x[map(i)]^2) + eps) * g
// One 256-thread block per row; sums of squares in fp32 with a fixed
// reduction tree, so a row's result never depends on the other rows.
#include "cb_internal.h"

namespace cb {

namespace {

// (packed: row i goes to the step-major layout of act_packed_index)
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const Tin* __restrict__ x, int n_src, const int* m1,
                                                      const int* m2, const float* __restrict__ g,
                                                      Tout* __restrict__ out, int d, float eps, int packed) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const int src = map_row(i, m1, m2);
  auto dst = [&](int c) { return out + (packed ? act_packed_index(i, c, d) : (int64_t)i * d + c); };
  if (src < 0 || src >= n_src) {  // invalid index: zero row, no out-of-bounds read
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) store8(dst(c), z);
    return;
  }
  const Tin* xr = x + (int64_t)src * d;
  float ss = 0.f;
  // d is a multiple of 8: each thread owns groups of 8 elements
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = sqrtf(tot / (float)d + eps);
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float v[8], gg[8], o[8];
    load8(xr + c, v);
    load8(g + c, gg);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (v[j] / rs) * gg[j];
    store8(dst(c), o);
  }
}

}  // namespace

hipError_t launch_rmsnorm(int dtype, bool x_f32, const void* x, int n_src, const int* m1, const int* m2,
                          const float* g, void* out, int rows, int d, float eps, hipStream_t s, bool packed_out) {
  if (rows <= 0) return hipSuccess;
  if (packed_out && (dtype != CB_BF16 || d % 32)) return hipErrorInvalidValue;
  const int pk = packed_out ? 1 : 0;
  LaunchScope ls("rmsnorm", s);
  if (dtype == CB_BF16) {
    if (x_f32)
      rmsnorm_kernel<float, bf16_t>
          <<<rows, 256, 0, s>>>((const float*)x, n_src, m1, m2, g, (bf16_t*)out, d, eps, pk);
    else
      rmsnorm_kernel<bf16_t, bf16_t>
          <<<rows, 256, 0, s>>>((const bf16_t*)x, n_src, m1, m2, g, (bf16_t*)out, d, eps, pk);
  } else {
    rmsnorm_kernel<float, float><<<rows, 256, 0, s>>>((const float*)x, n_src, m1, m2, g, (float*)out, d, eps, 0);
  }
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void iota_kernel(int* __restrict__ out, int n, int start) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = start + i;
}

}  // namespace

hipError_t launch_iota(int* out, int n, int start, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  LaunchScope ls("iota", s);
  iota_kernel<<<(n + 255) / 256, 256, 0, s>>>(out, n, start);
  return hipGetLastError();
}

}  // namespace cb
