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
//
// Per-block ranges (one lo, hi per 2048-key block of a channel): a block that
// holds no key before the call takes the range of the block before it,
// widened to cover the keys the call puts in it (block 0: those keys' own
// min and max); blocks that already hold keys keep theirs.  Since each new
// block's range is its predecessor's widened, block b's range is the running
// min/max over the new blocks up to b, started from the last old block's:
// append_range_kernel takes each new block's min/max, append_widen_kernel
// the running min/max (folded into the first kernel when the call starts one
// block).  The codes are then written as above, with each word's block range.
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
                                                    const float *__restrict__ hi, int64_t rs,
                                                    uint32_t *__restrict__ clamped) {
  const int c = threadIdx.x, h = blockIdx.y;
  const int64_t w = n_old / 32 + blockIdx.x;
  const int64_t i0 = w * 32 > n_old ? w * 32 : n_old;
  const int64_t i1 = w * 32 + 32 < n_old + m ? w * 32 + 32 : n_old + m;
  // the 32 keys of word w lie in 2048-key block w / 64
  const int64_t ro = rs == 0 ? (int64_t)h * kD + c : ((int64_t)h * rs + w / 64) * kD + c;
  const float l = lo[ro], u = hi[ro];
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

// Min/max of the new keys in block b0 + blockIdx.x (every key of a block the
// call starts is new) for kv head blockIdx.y: thread (r, c) takes rows r,
// r + 2, ... of channel c.  fold: the call starts this one block only, and
// the kernel also widens the previous block's range by it.  Stored ends are
// +0 for -0, as in the pack.
constexpr int kRangeThreads = 2 * kD;

template <typename T>
__global__ __launch_bounds__(kRangeThreads) void append_range_kernel(
    const T *__restrict__ keys, int64_t m, int64_t stride_tok, int64_t stride_head,
    int64_t n_old, int64_t b0, float *__restrict__ lo, float *__restrict__ hi, int64_t rs,
    int32_t fold) {
  const int c = threadIdx.x % kD, r = threadIdx.x / kD, h = blockIdx.y;
  const int64_t b = b0 + blockIdx.x;
  const int64_t i0 = b * kBlockKeys;
  const int64_t i1 = i0 + kBlockKeys < n_old + m ? i0 + kBlockKeys : n_old + m;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t i = i0 + r; i < i1; i += 2) {
    const float x = widen(keys[(i - n_old) * stride_tok + (int64_t)h * stride_head + c]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  __shared__ float2 red[kD];
  if (r == 1) red[c] = make_float2(mn, mx);
  __syncthreads();
  if (r != 0) return;
  mn = fminf(mn, red[c].x);
  mx = fmaxf(mx, red[c].y);
  const int64_t o = ((int64_t)h * rs + b) * kD + c;
  if (fold && b > 0) {
    mn = fminf(mn, lo[o - kD]);
    mx = fmaxf(mx, hi[o - kD]);
  }
  lo[o] = __fadd_rn(mn, 0.0f);
  hi[o] = __fadd_rn(mx, 0.0f);
}

// Running min/max over the blocks b0 .. b1-1 the call starts, from block
// b0 - 1's range (one thread per (kv head, channel), blocks in order).
__global__ __launch_bounds__(kD) void append_widen_kernel(int64_t b0, int64_t b1,
                                                          float *__restrict__ lo,
                                                          float *__restrict__ hi, int64_t rs) {
  const int c = threadIdx.x, h = blockIdx.x;
  float *lrow = lo + (int64_t)h * rs * kD + c, *hrow = hi + (int64_t)h * rs * kD + c;
  float mn = b0 > 0 ? lrow[(b0 - 1) * kD] : INFINITY;
  float mx = b0 > 0 ? hrow[(b0 - 1) * kD] : -INFINITY;
  for (int64_t b = b0; b < b1; ++b) {
    mn = fminf(mn, lrow[b * kD]);
    mx = fmaxf(mx, hrow[b * kD]);
    lrow[b * kD] = __fadd_rn(mn, 0.0f);
    hrow[b * kD] = __fadd_rn(mx, 0.0f);
  }
}

}  // namespace

int32_t launch_append(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                      int64_t stride_tok, int64_t stride_head, int64_t n_old,
                      uint32_t *planes, int64_t W, float *lo, float *hi, int64_t rs,
                      uint32_t *clamped, hipStream_t s) {
  const bool f16 = dtype == FATHOM_F16;
  if (rs > 0) {
    // ranges of the blocks this call starts
    const int64_t b0 = (n_old + kBlockKeys - 1) / kBlockKeys;
    const int64_t b1 = (n_old + m + kBlockKeys - 1) / kBlockKeys;
    if (b1 > b0) {
      const dim3 grid((unsigned)(b1 - b0), (unsigned)hkv);
      const int32_t fold = b1 - b0 == 1;
      if (f16)
        hipLaunchKernelGGL(append_range_kernel<__half>, grid, dim3(kRangeThreads), 0, s,
                           static_cast<const __half *>(keys), m, stride_tok, stride_head, n_old,
                           b0, lo, hi, rs, fold);
      else
        hipLaunchKernelGGL(append_range_kernel<float>, grid, dim3(kRangeThreads), 0, s,
                           static_cast<const float *>(keys), m, stride_tok, stride_head, n_old,
                           b0, lo, hi, rs, fold);
      if (!fold)
        hipLaunchKernelGGL(append_widen_kernel, dim3(hkv), dim3(kD), 0, s, b0, b1, lo, hi, rs);
    }
  }
  const int64_t words = (n_old + m - 1) / 32 - n_old / 32 + 1;
  const dim3 grid((unsigned)words, (unsigned)hkv);
  if (f16)
    hipLaunchKernelGGL(append_kernel<__half>, grid, dim3(kD), 0, s,
                       static_cast<const __half *>(keys), m, stride_tok, stride_head, n_old,
                       planes, W, lo, hi, rs, clamped);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(kD), 0, s,
                       static_cast<const float *>(keys), m, stride_tok, stride_head, n_old,
                       planes, W, lo, hi, rs, clamped);
  return hip_fail(hipGetLastError(), "append launch");
}

}  // namespace fathom
