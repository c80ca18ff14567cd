// Decode-time growth of a packed layer (explainer, deployment warnings item 3
// and the storage-cost line of 关键实验与数据: the planes are the stored
// 4-bit K, reused as keys arrive).  New keys are quantised with the layer's
// stored range and their bits written into plane rows with spare capacity.
//
// Grid (words, kv heads), kD threads: thread c of block (w, h) owns plane
// word w of the four planes of channel c, i.e. keys 32w .. 32w+31, so words
// shared with earlier tokens are rewritten by one thread (no atomics): the
// bits of the new keys are replaced, every other bit kept.  Key loads are
// coalesced across the block's channels.
#include <hip/hip_fp16.h>

#include "fathom_internal.h"

namespace fathom {
namespace {

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(__half x) { return __half2float(x); }

template <typename T>
__global__ __launch_bounds__(kD) void append_kernel(const T *__restrict__ keys, int64_t m,
                                                    int64_t stride_tok, int64_t stride_head,
                                                    int64_t n_old, uint32_t *__restrict__ planes,
                                                    int64_t W, const float *__restrict__ lo,
                                                    const float *__restrict__ hi,
                                                    uint32_t *__restrict__ clamped) {
  const int c = threadIdx.x, h = blockIdx.y;
  const int64_t w = n_old / 32 + blockIdx.x;
  const int64_t i0 = w * 32 > n_old ? w * 32 : n_old;
  const int64_t i1 = w * 32 + 32 < n_old + m ? w * 32 + 32 : n_old + m;
  const float l = lo[h * kD + c], u = hi[h * kD + c];
  const float delta = __fmul_rn(__fsub_rn(u, l), 0.0625f);
  uint32_t bits[kPlanes] = {0u, 0u, 0u, 0u};
  uint32_t mask = 0u, cnt = 0u;
  for (int64_t i = i0; i < i1; ++i) {
    const float x = widen(keys[(i - n_old) * stride_tok + (int64_t)h * stride_head + c]);
    int code = 0;
    if (delta != 0.0f) {
      const float fl = floorf(__fdiv_rn(__fsub_rn(x, l), delta));
      code = fl < 0.0f ? 0 : (fl > 15.0f ? 15 : (int)fl);
    }
    cnt += (x < l || x > u) ? 1u : 0u;
    const int b = (int)(i & 31);
    mask |= 1u << b;
#pragma unroll
    for (int s = 0; s < kPlanes; ++s) bits[s] |= (uint32_t)((code >> (3 - s)) & 1) << b;
  }
  uint32_t *pw = planes + ((int64_t)h * kD + c) * kPlanes * W + w;
#pragma unroll
  for (int s = 0; s < kPlanes; ++s) pw[s * W] = (pw[s * W] & ~mask) | bits[s];
  if (clamped) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((c & 63) == 0 && cnt) atomicAdd(clamped, cnt);
  }
}

}  // namespace

int32_t launch_append(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                      int64_t stride_tok, int64_t stride_head, int64_t n_old,
                      uint32_t *planes, int64_t W, const float *lo, const float *hi,
                      uint32_t *clamped, hipStream_t s) {
  const int64_t words = (n_old + m - 1) / 32 - n_old / 32 + 1;
  const dim3 grid((unsigned)words, (unsigned)hkv);
  if (dtype == FATHOM_F16)
    hipLaunchKernelGGL(append_kernel<__half>, grid, dim3(kD), 0, s,
                       static_cast<const __half *>(keys), m, stride_tok, stride_head, n_old,
                       planes, W, lo, hi, clamped);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(kD), 0, s,
                       static_cast<const float *>(keys), m, stride_tok, stride_head, n_old,
                       planes, W, lo, hi, clamped);
  return hip_fail(hipGetLastError(), "append launch");
}

}  // namespace fathom
