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

// Scan-traffic probe: the bytes an HBM-resident logits scan moves, with none
// of its arithmetic.  Block j of kv head g takes 2048-key tiles j, j + B, ...
// like the scan; per tile, wave w reads channels w, w + 16, ... with a quarter
// wave per plane slot (16-byte lanes, 256 bytes per plane row) for the plane
// slots below the channel's depth, and the block then writes rows_out fp32
// rows of the tile.  Depths are clamped to 0..4, so any depth table stays in
// bounds.
__global__ __launch_bounds__(1024) void probe_scan_traffic_kernel(
    const uint32_t *__restrict__ planes, int64_t W, int32_t hkv,
    const uint8_t *__restrict__ depth, int32_t rows_out, float *__restrict__ out, int64_t ld,
    uint32_t *__restrict__ sink) {
  const int g = blockIdx.x % hkv, j = blockIdx.x / hkv, bph = gridDim.x / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = lane >> 4, m16 = lane & 15;
  const int64_t ntiles = W / 64;
  const uint32_t *gp = planes + (int64_t)g * kD * kPlanes * W;
  int64_t off[8];
  bool on[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = wave + 16 * u;
    const int dep = min((int)depth[g * kD + c], kPlanes);
    on[u] = slot < dep;
    off[u] = (int64_t)(c * kPlanes + slot) * W + 4 * m16;
  }
  uint32_t acc = 0;
  for (int64_t t = j; t < ntiles; t += bph) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = on[u] ? *reinterpret_cast<const uint4 *>(gp + off[u] + 64 * t) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    const float f = __uint_as_float(acc & 0x007FFFFFu);
    for (int e = 4 * (int)threadIdx.x; e < rows_out * 2048; e += 4096) {
      const int r = e >> 11, k = e & 2047;
      *reinterpret_cast<float4 *>(out + (int64_t)(g * rows_out + r) * ld + 2048 * t + k) =
          make_float4(f, f, f, f);
    }
  }
  if (acc == 0x9E3779B9u) atomicXor(sink, acc);  // almost never taken; keeps the loads
}

}  // namespace

int32_t launch_probe_scan_traffic(const uint32_t *planes, int64_t n, int32_t hkv,
                                  const uint8_t *depth, int32_t rows_out, float *out,
                                  int64_t ld, uint32_t *sink, hipStream_t s) {
  const int blocks = max(1, device_cus() / hkv) * hkv;
  hipLaunchKernelGGL(probe_scan_traffic_kernel, dim3(blocks), dim3(1024), 0, s, planes, n / 32,
                     hkv, depth, rows_out, out, ld, sink);
  return hip_fail(hipGetLastError(), "probe launch");
}

int32_t launch_probe_read(const void *src, int64_t bytes, uint32_t *out, int32_t blocks,
                          hipStream_t s) {
  if (blocks == 0) blocks = device_cus() * 8;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const uint4 *>(src), bytes / 16, out);
  return hip_fail(hipGetLastError(), "probe launch");
}

}  // namespace fathom
