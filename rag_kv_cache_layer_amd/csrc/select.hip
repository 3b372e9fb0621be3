// HKVD selection: per-token K deviation and top-k.
//
// CacheBlend (arXiv 2405.16444) section 4.1 defines the KV deviation of
// token j on a layer as the difference between its reused and its fully
// recomputed KV; section 4.3 keeps the tokens with the highest deviation and,
// with gradual filtering (Figure 9), ranks only the tokens recomputed on the
// layer.  Here the deviation is the squared L2 norm of new minus cached K over
// all KV heads, summed from per-tile partials written by the QKV GEMM
// epilogue in a fixed order, and the ranking is (deviation descending, index
// ascending) with the kept set emitted in ascending index order.
//
// One 1024-thread workgroup: an MSB-first radix select over the 32-bit
// order-preserving key of each deviation (four 8-bit digits, LDS histograms
// with integer atomics, so the threshold is exact and deterministic), then a
// stable compaction by block-wide prefix sums.  Query rows are appended.
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Order-preserving key of a float: larger float -> larger unsigned key.
// -0 is folded onto +0 so that equal values tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the 1024 threads of the block.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    int x = lane < kSelWaves ? wave_tot[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      int t = __shfl_up(xi, o);
      if (lane >= o) xi += t;
    }
    if (lane < kSelWaves) wave_tot[lane] = xi - x;   // exclusive wave base
    if (lane == kSelWaves - 1) *total = xi;
  }
  __syncthreads();
  const int res = wave_tot[w] + incl - v;
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kSelWaves];
  __shared__ int s_total;
  __shared__ int s_bin, s_above;
  const int tid = threadIdx.x;
  // this workgroup's segment (one per request when several are batched)
  int in_off = 0, out_off = 0, n = a.n_cand, m_in = a.m_in, k_req = a.k;
  if (a.n_seg > 0) {
    const SelectArgs::Seg g = a.seg[blockIdx.x];
    in_off = g.in_off;
    out_off = g.out_off;
    n = g.n_cand;
    m_in = g.m_in;
    k_req = g.k;
  }
  float* const dev = a.dev + in_off;
  const int* const ids_in = a.ids_in ? a.ids_in + in_off : nullptr;
  int* const sel = a.sel ? a.sel + out_off : nullptr;
  int* const ids_out = a.ids_out ? a.ids_out + out_off : nullptr;

  // 1. deviation of every entry from the partial sums (fixed order)
  if (a.dev_part) {
    for (int i = tid; i < m_in; i += kSelThreads) {
      float s;
      if (i < n) {
        s = 0.f;
        for (int t = 0; t < a.n_parts; ++t) s += a.dev_part[(int64_t)t * a.ld_part + in_off + i];
      } else {
        s = __builtin_nanf("");
      }
      dev[i] = s;
    }
    __syncthreads();
  }

  const int n_query = m_in - n;
  // 2. nothing to drop: keep every entry
  if (k_req >= n) {
    for (int i = tid; i < m_in; i += kSelThreads) {
      if (sel) sel[i] = in_off + i;
      if (ids_out) ids_out[i] = ids_in ? ids_in[i] : i;
    }
    return;
  }
  const int k = k_req > 0 ? k_req : 0;

  // 3. radix select of the k-th largest key
  uint32_t prefix = 0, hmask = 0;
  int remaining = k;
  if (k > 0) {
    for (int sh = 24; sh >= 0; sh -= 8) {
      for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t key = order_key(dev[i]);
        if ((key & hmask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane L owns bins 255-4L .. 252-4L (descending)
        int c[4], local = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[255 - (4 * tid + j)];
          local += c[j];
        }
        int incl = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int t = __shfl_up(incl, o);
          if (tid >= o) incl += t;
        }
        const int excl = incl - local;
        if (excl < remaining && remaining <= incl) {
          int cum = excl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cum + c[j] >= remaining) {
              s_bin = 255 - (4 * tid + j);
              s_above = cum;
              break;
            }
            cum += c[j];
          }
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_bin << sh;
      hmask |= 255u << sh;
      remaining -= s_above;
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;      // key of the k-th largest deviation
  const int take_eq = remaining;    // how many keys equal to tau are kept (lowest indices)

  // 4. stable compaction in index order
  const int seg = (n + kSelThreads - 1) / kSelThreads;
  const int lo = min(n, tid * seg), hi = min(n, lo + seg);
  int c_eq = 0;
  if (k > 0)
    for (int i = lo; i < hi; ++i) c_eq += order_key(dev[i]) == tau;
  int eq_seen = block_exclusive_scan(c_eq, wave_tot, &s_total);
  int c_keep = 0;
  if (k > 0)
    for (int i = lo; i < hi; ++i) {
      const uint32_t key = order_key(dev[i]);
      if (key > tau) ++c_keep;
      else if (key == tau) { if (eq_seen < take_eq) ++c_keep; ++eq_seen; }
    }
  int out = block_exclusive_scan(c_keep, wave_tot, &s_total);
  if (k > 0) {
    eq_seen -= c_eq;  // back to this segment's base
    for (int i = lo; i < hi; ++i) {
      const uint32_t key = order_key(dev[i]);
      bool keep = key > tau;
      if (key == tau) { keep = eq_seen < take_eq; ++eq_seen; }
      if (keep) {
        if (sel) sel[out] = in_off + i;
        if (ids_out) ids_out[out] = ids_in ? ids_in[i] : i;
        ++out;
      }
    }
  }
  // 5. query rows, always kept, after the candidates
  for (int j = tid; j < n_query; j += kSelThreads) {
    const int i = n + j;
    if (sel) sel[k + j] = in_off + i;
    if (ids_out) ids_out[k + j] = ids_in ? ids_in[i] : i;
  }
}

// One wave per candidate row.
template <typename T>
__global__ __launch_bounds__(256) void kdev_kernel(const T* __restrict__ k_new, const T* __restrict__ k_ref,
                                                   const int* rows, int n, int kv_dim, int T_rows,
                                                   float* __restrict__ dev) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const int r = rows ? rows[i] : i;
  float s = 0.f;
  if (r >= 0 && r < T_rows) {
    // two 512-element steps per iteration: all four 16-byte loads are issued
    // before the arithmetic (same accumulation order as one step at a time)
    int c = lane * 8;
    for (; c + 512 < kv_dim; c += 2 * 512) {
      float x[2][8], y[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        load8(k_new + (int64_t)i * kv_dim + c + u * 512, x[u]);
        load8(k_ref + (int64_t)r * kv_dim + c + u * 512, y[u]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float d = x[u][j] - y[u][j];
          s += d * d;
        }
    }
    for (; c < kv_dim; c += 512) {
      float x[8], y[8];
      load8(k_new + (int64_t)i * kv_dim + c, x);
      load8(k_ref + (int64_t)r * kv_dim + c, y);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = x[j] - y[j];
        s += d * d;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) dev[i] = s;
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  LaunchScope ls("select_topk", s);
  select_kernel<<<a.n_seg > 0 ? a.n_seg : 1, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kdev(int dtype, const void* k_new, const void* k_ref, const int* rows, int n, int kv_dim,
                       int T, float* dev, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  LaunchScope ls("kdev", s);
  const int blocks = (n + 3) / 4;
  if (dtype == CB_BF16)
    kdev_kernel<bf16_t><<<blocks, 256, 0, s>>>((const bf16_t*)k_new, (const bf16_t*)k_ref, rows, n, kv_dim, T,
                                               dev);
  else
    kdev_kernel<float><<<blocks, 256, 0, s>>>((const float*)k_new, (const float*)k_ref, rows, n, kv_dim, T, dev);
  return hipGetLastError();
}

}  // namespace cb
