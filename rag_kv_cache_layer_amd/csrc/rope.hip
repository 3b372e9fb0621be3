// RoPE position re-alignment of cached keys, in place, over many layers.
//
// CacheBlend (arXiv 2405.16444) section 4.3, footnote 3: a chunk's keys were
// rotated at the positions the chunk had when it was prefilled alone; after
// it is placed at offset delta, one more rotation by delta*theta_i per pair
// moves every key to its absolute position (the aifetchly guide, "RoPE Delta
// Positional Realignment": R(m + delta) = R(delta) R(m)); values stay as they
// are.
//
// The kernel is HBM-bound: every shifted element is read once and written
// once.  One thread moves 16 consecutive elements (8 pairs) of one key row:
// two 16 B loads and stores for bf16, coalesced along the row; the cos/sin
// rows of the few distinct deltas stay in L2.
#include "cb_internal.h"

namespace cb {

namespace {

// 8-element units per thread: two (32 B in flight per thread) measure ~20%
// faster than one on a cold stack-wide launch and match a plain copy within 7%.
// A key row whose length is not a multiple of 8 * CB_ROPE_UPT elements (an
// fp32 layout such as one KV head of 72) takes one unit per thread instead.
#ifndef CB_ROPE_UPT
#define CB_ROPE_UPT 2
#endif

template <typename T, int UPT>
__global__ __launch_bounds__(256) void rope_shift_kernel(T* __restrict__ k, int64_t lstride, int kv_dim,
                                                         int hd, int row0, int n_rows, int units_per_row,
                                                         int64_t total, const float* __restrict__ cosp,
                                                         const float* __restrict__ sinp, ChunkOffsets offs,
                                                         int n_chunks) {
  int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= total) return;
  int cu = (int)(u % units_per_row);
  int64_t rr = u / units_per_row;
  int r = row0 + (int)(rr % n_rows);
  int l = (int)(rr / n_rows);
  const int cu0 = cu * UPT;   // this thread's first 8-element unit of the row
  const int delta = chunk_delta(offs, n_chunks, r);
  T* p = k + (int64_t)l * lstride + (int64_t)r * kv_dim + cu0 * 8;
  float v[UPT][8];
#pragma unroll
  for (int x = 0; x < UPT; ++x) load8(p + x * 8, v[x]);
#pragma unroll
  for (int x = 0; x < UPT; ++x) {
    const int e = ((cu0 + x) * 8) % hd;
    const float* cs = cosp + (int64_t)delta * (hd / 2) + e / 2;
    const float* sn = sinp + (int64_t)delta * (hd / 2) + e / 2;
    float o[8];
    rope_rotate8(v[x], cs, sn, o);
    store8(p + x * 8, o);
  }
}

}  // namespace

hipError_t launch_rope_shift(int dtype, const RopeShiftArgs& a, hipStream_t s) {
  if (a.n_chunks < 2 || a.n_layers <= 0) return hipSuccess;
  const int row0 = a.offsets[1];
  const int n_rows = a.offsets[a.n_chunks] - row0;
  if (n_rows <= 0) return hipSuccess;
  ChunkOffsets offs;
  for (int c = 0; c <= a.n_chunks; ++c) offs.o[c] = a.offsets[c];
  // kv_dim is a multiple of 8 (head_dim is); rows that do not split into
  // whole CB_ROPE_UPT-unit groups use one unit per thread
  const int upt = a.kv_dim % (8 * CB_ROPE_UPT) == 0 ? CB_ROPE_UPT : 1;
  const int upr = a.kv_dim / 8 / upt;   // threads per row
  const int64_t total = (int64_t)a.n_layers * n_rows * upr;
  const int64_t blocks = (total + 255) / 256;
  LaunchScope ls("rope_shift", s);
#define CB_ROPE_LAUNCH(T_, U_)                                                                                  \
  rope_shift_kernel<T_, U_><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(                                        \
      (T_*)a.k_cache, a.layer_stride, a.kv_dim, a.hd, row0, n_rows, upr, total, a.cos, a.sin, offs, a.n_chunks)
  if (dtype == CB_BF16) {
    if (upt == CB_ROPE_UPT) CB_ROPE_LAUNCH(bf16_t, CB_ROPE_UPT); else CB_ROPE_LAUNCH(bf16_t, 1);
  } else {
    if (upt == CB_ROPE_UPT) CB_ROPE_LAUNCH(float, CB_ROPE_UPT); else CB_ROPE_LAUNCH(float, 1);
  }
#undef CB_ROPE_LAUNCH
  return hipGetLastError();
}

}  // namespace cb
