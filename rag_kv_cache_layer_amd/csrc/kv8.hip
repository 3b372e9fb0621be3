// Stored 8-bit chunk KV expanded into the working cache, with the RoPE
// re-alignment of the keys fused in.
//
// The paper serves its larger models with 8-bit weights (CacheBlend section
// 7, models); the same E4M3 format with one power-of-two scale per (token,
// KV head) row of head_dim values halves the bytes of the stored chunk KV,
// which is what the loading path of section 5 moves from host memory or disk.
// Expansion is exact: an E4M3 value times a power of two is representable in
// fp32 and in bf16.  Keys of chunk c >= 1 are then rotated by delta = o_c
// (section 4.3, footnote 3) with the arithmetic of the in-place shift (two
// rounded fp32 products, one rounded sum, one rounding to the cache dtype),
// so expanding and shifting here gives the bits that expanding and then
// calling the in-place shift gives.
//
// HBM-bound: one byte per element read, two (bf16) or four (fp32) written.
// One thread expands 16 consecutive codes of one row (a 16-byte load).
#include "cb_internal.h"

namespace cb {

namespace {

struct KvOffsets {
  int32_t o[kMaxShiftChunks + 1];
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <typename T>
__global__ __launch_bounds__(256) void kv_expand_kernel(KvExpandArgs a, KvOffsets offs, int units_per_row,
                                                        int64_t total) {
  int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= 2 * total) return;
  const bool is_v = u >= total;
  if (is_v) u -= total;
  const int cu = (int)(u % units_per_row);
  const int64_t rr = u / units_per_row;
  const int rl = (int)(rr % a.n_rows);   // row within the expanded range
  const int l = (int)(rr / a.n_rows);
  const int r = a.row0 + rl;              // cache row
  const int col = cu * 16;
  const int head = col / a.hd;
  const int64_t code_row = (int64_t)l * a.n_rows + rl;
  const uint8_t* src = (is_v ? a.v_codes : a.k_codes) + code_row * a.kv_dim + col;
  const int e = (is_v ? a.v_exps : a.k_exps)[code_row * a.n_kv + head];
  const uint4 w = *reinterpret_cast<const uint4*>(src);
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  float v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], true);
    v[4 * q + 0] = ldexpf(lo[0], e);
    v[4 * q + 1] = ldexpf(lo[1], e);
    v[4 * q + 2] = ldexpf(hi[0], e);
    v[4 * q + 3] = ldexpf(hi[1], e);
  }
  if (!is_v && a.shift && a.n_chunks > 1 && r >= offs.o[1] && r < offs.o[a.n_chunks]) {
    // chunk of row r: the largest c in [1, n_chunks-1] with o[c] <= r
    int lo = 1, hi = a.n_chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs.o[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int delta = offs.o[lo];
    const int half = a.hd / 2;
    const float* cs = a.cos + (int64_t)delta * half + (col % a.hd) / 2;
    const float* sn = a.sin + (int64_t)delta * half + (col % a.hd) / 2;
    {
      // two rounded products and one rounded sum per output, as the shift
#pragma clang fp contract(off)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x0 = v[2 * j], x1 = v[2 * j + 1], c = cs[j], s = sn[j];
        v[2 * j] = x0 * c - x1 * s;
        v[2 * j + 1] = x0 * s + x1 * c;
      }
    }
  }
  T* dst = (T*)(is_v ? a.v_cache : a.k_cache) + (int64_t)l * a.layer_stride + (int64_t)r * a.kv_dim + col;
  store8(dst, v);
  store8(dst + 8, v + 8);
}

}  // namespace

hipError_t launch_kv_expand(int dtype, const KvExpandArgs& a, const int32_t* offsets, hipStream_t s) {
  if (a.n_layers <= 0 || a.n_rows <= 0) return hipSuccess;
  KvOffsets offs{};
  for (int c = 0; c <= a.n_chunks; ++c) offs.o[c] = offsets[c];
  const int upr = a.kv_dim / 16;
  const int64_t total = (int64_t)a.n_layers * a.n_rows * upr;
  const int64_t blocks = (2 * total + 255) / 256;
  LaunchScope ls("kv_expand", s);
  if (dtype == CB_BF16)
    kv_expand_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a, offs, upr, total);
  else
    kv_expand_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a, offs, upr, total);
  return hipGetLastError();
}

}  // namespace cb
