// Streaming-read probe: the bandwidth denominator for the scan's roofline.
// Every CU streams 16-byte loads over the buffer (HBM or pinned host memory,
// which is then read zero-copy over the host link) and folds them into one
// checksum word so the loads cannot be dropped.
#include "fathom_internal.h"

namespace fathom {
namespace {

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *__restrict__ src,
                                                         int64_t n16,
                                                         uint32_t *__restrict__ out) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * step < n16; i += 4 * step) {
    const uint4 a = src[i], b = src[i + step], c = src[i + 2 * step], d = src[i + 3 * step];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^
           d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += step) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) atomicXor(out, acc);  // almost never taken; keeps the loads
}

}  // namespace

int32_t launch_probe_read(const void *src, int64_t bytes, uint32_t *out, int32_t blocks,
                          hipStream_t s) {
  if (blocks == 0) blocks = device_cus() * 8;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const uint4 *>(src), bytes / 16, out);
  return hip_fail(hipGetLastError(), "probe launch");
}

}  // namespace fathom
