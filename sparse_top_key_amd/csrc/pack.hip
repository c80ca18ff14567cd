// Storage side of Fathom (explainer, section 核心方法, storage side): 4-bit
// per-channel min-max quantisation of K into channel-major bit planes.
//
//   pack_minmax   per-(chunk, kv head, channel) min / max partials
//   pack_range    reduce the partials -> lo, hi  (stored +0 for a -0 end)
//   pack_planes   codes -> 4 bit planes via wave64 ballots; per-block code
//                 sums S1, S2 from popcounts of the ballots (exact integers)
//   pack_sigma    sigma^2 = Var(code) * delta^2 from the exact integer sums
//
// Every value is bit-identical to the CPU definition: min/max are exact, the
// quantiser uses one IEEE fp32 subtract and one correctly rounded fp32 divide,
// and the variance is evaluated from exact int64 sums in a fixed fp64 order.
#include <hip/hip_fp16.h>

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kMinmaxThreads = 256;
constexpr int kPlaneThreads = 256;           // 4 waves, 32 channels each
constexpr int kSubTile = 64;                 // keys per ballot (one wave)
constexpr int kLdsPitch = kD + 1;            // fp32 words per staged key row

__device__ inline float load_key(const __half *p) { return __half2float(*p); }
__device__ inline float load_key(const float *p) { return *p; }

// Partial min/max of chunk blockIdx.x for kv head blockIdx.y.
template <typename T>
__global__ __launch_bounds__(kMinmaxThreads) void pack_minmax_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok,
    int64_t stride_head, int64_t chunk, float2 *__restrict__ part) {
  const int h = blockIdx.y;
  const int hkv = gridDim.y;
  const int c = threadIdx.x % kD;
  const int r = threadIdx.x / kD;  // 0..1
  const int64_t i0 = (int64_t)blockIdx.x * chunk;
  const int64_t i1 = min(n, i0 + chunk);
  float mn = INFINITY, mx = -INFINITY;
  const T *base = keys + (int64_t)h * stride_head + c;
  for (int64_t i = i0 + r; i < i1; i += kMinmaxThreads / kD) {
    float x = load_key(base + i * stride_tok);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  __shared__ float2 red[kMinmaxThreads];
  red[threadIdx.x] = make_float2(mn, mx);
  __syncthreads();
  if (r == 0) {
    float2 o = red[threadIdx.x + kD];
    mn = fminf(mn, o.x);
    mx = fmaxf(mx, o.y);
    part[((int64_t)blockIdx.x * hkv + h) * kD + c] = make_float2(mn, mx);
  }
}

__global__ __launch_bounds__(kD) void pack_range_kernel(
    const float2 *__restrict__ part, int32_t nparts, int32_t hkv,
    float *__restrict__ lo, float *__restrict__ hi) {
  const int h = blockIdx.x, c = threadIdx.x;
  float mn = INFINITY, mx = -INFINITY;
  for (int p = 0; p < nparts; ++p) {
    float2 v = part[((int64_t)p * hkv + h) * kD + c];
    mn = fminf(mn, v.x);
    mx = fmaxf(mx, v.y);
  }
  // -0 and +0 are one key value: the stored ends are +0.
  lo[h * kD + c] = __fadd_rn(mn, 0.0f);
  hi[h * kD + c] = __fadd_rn(mx, 0.0f);
}

__device__ inline int quantise(float x, float lo, float delta) {
  if (delta == 0.0f) return 0;
  float y = __fdiv_rn(__fsub_rn(x, lo), delta);
  float f = floorf(y);
  return f > 15.0f ? 15 : (int)f;
}

// One block = 2048 keys (one 64-word block of every plane row) of kv head
// blockIdx.y.  Keys are staged 64 at a time through LDS (coalesced rows),
// then each wave turns one channel column into 4 ballots (64 keys = two
// plane words per plane) for its 32 channels.
template <typename T>
__global__ __launch_bounds__(kPlaneThreads) void pack_planes_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok,
    int64_t stride_head, int64_t W, const float *__restrict__ lo,
    const float *__restrict__ hi, uint32_t *__restrict__ planes,
    int2 *__restrict__ sums) {
  __shared__ float tile[kSubTile * kLdsPitch];
  const int h = blockIdx.y;
  const int hkv = gridDim.y;
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t key0 = (int64_t)blockIdx.x * kBlockKeys;

  // lane cc of this wave keeps channel (wave*32 + cc)'s range and sums
  const int my_c = wave * 32 + (lane & 31);
  const float my_lo = lo[h * kD + my_c];
  const float my_delta = __fmul_rn(__fsub_rn(hi[h * kD + my_c], my_lo), 0.0625f);
  int my_s1 = 0, my_s2 = 0;

  for (int sub = 0; sub < kBlockKeys / kSubTile; ++sub) {
    const int64_t kb = key0 + sub * kSubTile;
    __syncthreads();
    for (int e = threadIdx.x; e < kSubTile * kD; e += kPlaneThreads) {
      const int t = e / kD, c = e % kD;
      const int64_t i = kb + t;
      tile[t * kLdsPitch + c] =
          i < n ? load_key(keys + i * stride_tok + (int64_t)h * stride_head + c)
                : 0.0f;
    }
    __syncthreads();
    const bool valid = kb + lane < n;
    const int64_t w0 = kb / 32;
#pragma unroll 4
    for (int cc = 0; cc < 32; ++cc) {
      const int c = wave * 32 + cc;
      const float clo = __shfl(my_lo, cc);
      const float cdelta = __shfl(my_delta, cc);
      const int code = valid ? quantise(tile[lane * kLdsPitch + c], clo, cdelta) : 0;
      const uint64_t m0 = __ballot(code & 1);
      const uint64_t m1 = __ballot(code & 2);
      const uint64_t m2 = __ballot(code & 4);
      const uint64_t m3 = __ballot(code & 8);
      // lanes 0..7 store slot s = lane/2 (bit 3 - s), word half lane%2
      if (lane < 8) {
        const int s = lane >> 1;
        const uint64_t m = s == 0 ? m3 : s == 1 ? m2 : s == 2 ? m1 : m0;
        const uint32_t word = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
        planes[(((int64_t)h * kD + c) * kPlanes + s) * W + w0 + (lane & 1)] = word;
      }
      // S1 = sum code, S2 = sum code^2 from popcounts of the bit planes
      const int p0 = __popcll(m0), p1 = __popcll(m1), p2 = __popcll(m2),
                p3 = __popcll(m3);
      const int s1 = p0 + 2 * p1 + 4 * p2 + 8 * p3;
      const int s2 = p0 + 4 * p1 + 16 * p2 + 64 * p3 +
                     2 * (2 * __popcll(m0 & m1) + 4 * __popcll(m0 & m2) +
                          8 * __popcll(m0 & m3) + 8 * __popcll(m1 & m2) +
                          16 * __popcll(m1 & m3) + 32 * __popcll(m2 & m3));
      if ((lane & 31) == cc) {
        my_s1 += s1;
        my_s2 += s2;
      }
    }
  }
  if (lane < 32)
    sums[((int64_t)blockIdx.x * hkv + h) * kD + my_c] = make_int2(my_s1, my_s2);
}

__global__ __launch_bounds__(kD) void pack_sigma_kernel(
    const int2 *__restrict__ sums, int32_t nblocks, int32_t hkv, int64_t n,
    const float *__restrict__ lo, const float *__restrict__ hi,
    float *__restrict__ sigma2) {
  const int h = blockIdx.x, c = threadIdx.x;
  int64_t s1 = 0, s2 = 0;
  for (int b = 0; b < nblocks; ++b) {
    int2 v = sums[((int64_t)b * hkv + h) * kD + c];
    s1 += v.x;
    s2 += v.y;
  }
  const float l = lo[h * kD + c];
  const float delta = __fmul_rn(__fsub_rn(hi[h * kD + c], l), 0.0625f);
  const int64_t num = n * s2 - s1 * s1;
  const double var_code = __ddiv_rn((double)num, __dmul_rn((double)n, (double)n));
  const double dd = __dmul_rn((double)delta, (double)delta);
  sigma2[h * kD + c] = (float)__dmul_rn(var_code, dd);
}

struct PackLayout {
  int64_t chunk;
  int32_t nparts;
  int32_t nblocks;
  int64_t part_bytes;
  int64_t sums_bytes;
};

PackLayout pack_layout(int64_t n, int32_t hkv) {
  PackLayout L;
  // enough min/max blocks to fill the chip, each at least 256 keys
  int64_t parts = (2048 + hkv - 1) / hkv;
  parts = std::min<int64_t>(parts, (n + 255) / 256);
  parts = std::max<int64_t>(parts, 1);
  L.chunk = (n + parts - 1) / parts;
  L.nparts = (int32_t)((n + L.chunk - 1) / L.chunk);
  L.nblocks = (int32_t)(plane_words(n) / 64);
  L.part_bytes = ((int64_t)L.nparts * hkv * kD * sizeof(float2) + 255) / 256 * 256;
  L.sums_bytes = (int64_t)L.nblocks * hkv * kD * sizeof(int2);
  return L;
}

template <typename T>
int32_t launch_pack_t(const T *keys, int64_t n, int32_t hkv, int64_t stride_tok,
                      int64_t stride_head, uint32_t *planes, float *lo,
                      float *hi, float *sigma2, void *ws, hipStream_t s) {
  const PackLayout L = pack_layout(n, hkv);
  float2 *part = reinterpret_cast<float2 *>(ws);
  int2 *sums = reinterpret_cast<int2 *>(static_cast<char *>(ws) + L.part_bytes);
  const int64_t W = plane_words(n);
  hipLaunchKernelGGL(pack_minmax_kernel<T>, dim3(L.nparts, hkv), dim3(kMinmaxThreads),
                     0, s, keys, n, stride_tok, stride_head, L.chunk, part);
  hipLaunchKernelGGL(pack_range_kernel, dim3(hkv), dim3(kD), 0, s, part, L.nparts,
                     hkv, lo, hi);
  hipLaunchKernelGGL(pack_planes_kernel<T>, dim3(L.nblocks, hkv), dim3(kPlaneThreads),
                     0, s, keys, n, stride_tok, stride_head, W, lo, hi, planes, sums);
  hipLaunchKernelGGL(pack_sigma_kernel, dim3(hkv), dim3(kD), 0, s, sums, L.nblocks,
                     hkv, n, lo, hi, sigma2);
  return hip_fail(hipGetLastError(), "pack launch");
}

}  // namespace

int64_t pack_workspace_bytes(int64_t n, int32_t hkv) {
  const PackLayout L = pack_layout(n, hkv);
  return L.part_bytes + L.sums_bytes;
}

int32_t launch_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                    int64_t stride_tok, int64_t stride_head, uint32_t *planes,
                    float *lo, float *hi, float *sigma2, void *ws, hipStream_t s) {
  if (dtype == FATHOM_F16)
    return launch_pack_t(static_cast<const __half *>(keys), n, hkv, stride_tok,
                         stride_head, planes, lo, hi, sigma2, ws, s);
  return launch_pack_t(static_cast<const float *>(keys), n, hkv, stride_tok,
                       stride_head, planes, lo, hi, sigma2, ws, s);
}

}  // namespace fathom
