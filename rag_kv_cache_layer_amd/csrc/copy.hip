// A plain streaming copy: the measured HBM ceiling for the bandwidth-bound
// kernels of the fusor (the RoPE shift, the K deviation, the scatter, the
// 8-bit KV expansion), which each read and/or write every byte once.
//
// Every wave instruction moves 1 KB of contiguous memory (thread t of a
// workgroup takes 16-byte unit t of a 4 KB block); a workgroup moves IL
// blocks with all its loads issued before its stores, and the stores are
// non-temporal (the copy's output is not read back soon, so it should not
// displace cached data).  On MI355X this streams faster than hipMemcpy's
// device-to-device kernel.
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kCopyIL = 4;

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                          int64_t n) {
  const int64_t first = (int64_t)blockIdx.x * 256 * kCopyIL + threadIdx.x;
  u32x4_t v[kCopyIL];
#pragma unroll
  for (int x = 0; x < kCopyIL; ++x) {
    const int64_t i = first + (int64_t)x * 256;
    if (i < n) v[x] = src[i];
  }
#pragma unroll
  for (int x = 0; x < kCopyIL; ++x) {
    const int64_t i = first + (int64_t)x * 256;
    if (i < n) __builtin_nontemporal_store(v[x], &dst[i]);
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 256 * kCopyIL - 1) / (256 * kCopyIL);
  LaunchScope ls("stream_copy", s);
  stream_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((const u32x4_t*)src, (u32x4_t*)dst, n);
  return hipGetLastError();
}

}  // namespace cb
