// Sparse decode attention over the selected keys: the step after the top-k
// (explainer, problem statement: each generated token attends over the top k
// of the n keys; future-work list: V stays dense).  The pages give no layout
// for it; here K and V are full-precision token-major rows, in HBM or pinned
// host memory, gathered by index.
//
//   s_i = scale * q . K_i,  p_i = exp(s_i - m),  out = sum p_i V_i / sum p_i,
//   lse = m + log(sum p_i)  over the listed keys of each row.
//
// Two launches.  attn_partial_kernel: a 256-thread block takes 256 entries of
// one index row; each wave owns 64 entries and produces a partial
// (m, l, o[128]) per query head of the row.  Lane j scores entry j from its
// own K row (16-byte loads, q broadcast from LDS); the wave's 64 V rows are
// then read row by row, one coalesced 256-byte row per instruction, a batch
// of them (64 fp16 rows, 32 fp32 rows) issued before the first use, so
// host-resident rows overlap their latency.
// attn_combine_kernel merges the partials of a head by their maxima.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnBlockKeys = kAttnWaves * 64;
constexpr int kPart = kD + 2;  // m, l, o[0..127]

// Element access: a K row is kD / kPerVec 16-byte vectors; a lane's share of
// a V row is the pair of channels 2l, 2l+1.
template <typename T>
struct Elem;
template <>
struct Elem<_Float16> {
  static constexpr int kPerVec = 8;
  __device__ static void cvt(uint4 u, float (&f)[kPerVec]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
  using Pair = uint32_t;
  __device__ static void unpair(Pair v, float &a, float &b) {
    a = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
    b = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static void cvt(uint4 u, float (&f)[kPerVec]) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  using Pair = float2;
  __device__ static void unpair(Pair v, float &a, float &b) {
    a = v.x;
    b = v.y;
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = __fadd_rn(v, __shfl_xor(v, off));
  return v;
}

// grid (ceil(k / 256), rows); row r serves query heads r*GH .. r*GH+GH-1.
// part[((r * nparts + wave_index) * GH + j) * kPart + ...]
template <typename T, int GH>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(
    const float *__restrict__ q, int32_t heads_per_kv, const T *__restrict__ kc,
    const T *__restrict__ vc, int64_t n, int64_t stride_tok, int64_t stride_head,
    const int32_t *__restrict__ idx, int32_t k, float scale, float *__restrict__ part,
    int32_t nparts) {
  __shared__ float s_q[GH][kD];
  const int r = blockIdx.y;
  const int h0 = r * GH;
  const int g = h0 / heads_per_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < GH * kD; e += kAttnThreads) s_q[e / kD][e % kD] = q[(int64_t)h0 * kD + e];
  __syncthreads();

  const int j = blockIdx.x * kAttnBlockKeys + wave * 64 + lane;
  int key = -1;
  if (j < k) {
    const int v = idx[(int64_t)r * k + j];
    key = (v >= 0 && v < n) ? v : -1;  // padding and out-of-range entries are skipped
  }
  const int64_t head_off = (int64_t)g * stride_head;
  const bool any = __ballot(key >= 0) != 0ull;

  using E = Elem<T>;
  using Pair = typename E::Pair;
  constexpr int kVecs = kD / E::kPerVec;  // 16-byte vectors per K row
  constexpr int kKChunk = 16;              // vectors in flight per lane
  constexpr int kVBatch = 256 / sizeof(Pair);  // V rows in flight per wave

  // ---- scores: lane j scores its own entry ---------------------------------
  float dot[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) dot[h] = 0.0f;
  if (key >= 0) {
    const uint4 *kr = reinterpret_cast<const uint4 *>(kc + (int64_t)key * stride_tok + head_off);
#pragma unroll
    for (int c0 = 0; c0 < kVecs; c0 += kKChunk) {
      uint4 raw[kKChunk];
#pragma unroll
      for (int v = 0; v < kKChunk; ++v) raw[v] = kr[c0 + v];
#pragma unroll
      for (int v = 0; v < kKChunk; ++v) {
        float f[E::kPerVec];
        E::cvt(raw[v], f);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e)
#pragma unroll
          for (int h = 0; h < GH; ++h)
            dot[h] = fmaf(s_q[h][(c0 + v) * E::kPerVec + e], f[e], dot[h]);
      }
    }
  }

  float m[GH], p[GH], l[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const float sc = key >= 0 ? __fmul_rn(scale, dot[h]) : -INFINITY;
    m[h] = wave_max(sc);
    p[h] = key >= 0 ? expf(__fsub_rn(sc, m[h])) : 0.0f;
    l[h] = wave_sum(p[h]);
  }

  // ---- o = sum_j p_j V_j over the wave's entries, in entry order -----------
  // lane l holds channels 2l, 2l+1; a skipped entry reads row 0 with weight 0
  float o0[GH], o1[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) o0[h] = o1[h] = 0.0f;
  if (any) {
#pragma unroll
    for (int j0 = 0; j0 < 64; j0 += kVBatch) {
      Pair vr[kVBatch];
#pragma unroll
      for (int jj = 0; jj < kVBatch; ++jj) {
        const int kj = __builtin_amdgcn_readlane(key, j0 + jj);
        const int64_t row = kj >= 0 ? kj : 0;
        vr[jj] = *reinterpret_cast<const Pair *>(vc + row * stride_tok + head_off + 2 * lane);
      }
#pragma unroll
      for (int jj = 0; jj < kVBatch; ++jj) {
        float a, b;
        E::unpair(vr[jj], a, b);
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float pj =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[h]), j0 + jj));
          o0[h] = fmaf(pj, a, o0[h]);
          o1[h] = fmaf(pj, b, o1[h]);
        }
      }
    }
  }
  const int pi = blockIdx.x * kAttnWaves + wave;
  if (pi < nparts) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float *dst = part + ((int64_t)(r * nparts + pi) * GH + h) * kPart;
      if (lane == 0) {
        dst[0] = m[h];
        dst[1] = l[h];
      }
      dst[2 + 2 * lane] = o0[h];
      dst[3 + 2 * lane] = o1[h];
    }
  }
}

// One block of kD threads per query head h (idx row h / GH, head h % GH).
template <int GH>
__global__ __launch_bounds__(kD) void attn_combine_kernel(const float *__restrict__ part,
                                                          int32_t nparts,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int h = blockIdx.x, c = threadIdx.x;
  const int r = h / GH, hh = h % GH;
  const float *base = part + ((int64_t)r * nparts * GH + hh) * kPart;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, base[(int64_t)i * GH * kPart]);
  float L = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
    for (int i = 0; i < nparts; ++i) {
      const float *pp = base + (int64_t)i * GH * kPart;
      const float mi = pp[0];
      if (mi == -INFINITY) continue;
      const float w = expf(__fsub_rn(mi, M));
      L = fmaf(w, pp[1], L);
      o = fmaf(w, pp[2 + c], o);
    }
  }
  out[(int64_t)h * kD + c] = L > 0.0f ? __fdiv_rn(o, L) : 0.0f;
  if (c == 0) lse[h] = L > 0.0f ? __fadd_rn(M, logf(L)) : -INFINITY;
}

template <typename T, int GH>
int32_t launch_attn_t(const float *q, int32_t hq, int32_t hkv, const void *kc, const void *vc,
                      int64_t n, int64_t stride_tok, int64_t stride_head, const int32_t *idx,
                      int32_t k, float scale, float *out, float *lse, void *ws, hipStream_t s) {
  const int32_t rows = hq / GH;
  const int32_t nparts = (k + 63) / 64;
  float *part = static_cast<float *>(ws);
  if (nparts > 0) {
    const dim3 grid((k + kAttnBlockKeys - 1) / kAttnBlockKeys, rows);
    hipLaunchKernelGGL((attn_partial_kernel<T, GH>), grid, dim3(kAttnThreads), 0, s, q, hq / hkv,
                       static_cast<const T *>(kc), static_cast<const T *>(vc), n, stride_tok,
                       stride_head, idx, k, scale, part, nparts);
  }
  hipLaunchKernelGGL((attn_combine_kernel<GH>), dim3(hq), dim3(kD), 0, s, part, nparts, out, lse);
  return hip_fail(hipGetLastError(), "sparse_attention launch");
}

template <typename T>
int32_t launch_attn_dtype(int32_t group, const float *q, int32_t hq, int32_t hkv, const void *kc,
                          const void *vc, int64_t n, int64_t st, int64_t sh, const int32_t *idx,
                          int32_t k, float scale, float *out, float *lse, void *ws,
                          hipStream_t s) {
  switch (group) {
    case 1: return launch_attn_t<T, 1>(q, hq, hkv, kc, vc, n, st, sh, idx, k, scale, out, lse, ws, s);
    case 2: return launch_attn_t<T, 2>(q, hq, hkv, kc, vc, n, st, sh, idx, k, scale, out, lse, ws, s);
    case 4: return launch_attn_t<T, 4>(q, hq, hkv, kc, vc, n, st, sh, idx, k, scale, out, lse, ws, s);
    default: return launch_attn_t<T, 8>(q, hq, hkv, kc, vc, n, st, sh, idx, k, scale, out, lse, ws, s);
  }
}

}  // namespace

int64_t attn_workspace_bytes(int32_t hq, int32_t k) {
  return (int64_t)hq * ((k + 63) / 64) * kPart * (int64_t)sizeof(float);
}

int32_t launch_attention(const float *q, int32_t hq, int32_t hkv, const void *kc, const void *vc,
                         int32_t dtype, int64_t n, int64_t stride_tok, int64_t stride_head,
                         const int32_t *idx, int32_t group, int32_t k, float scale, float *out,
                         float *lse, void *ws, hipStream_t s) {
  if (dtype == FATHOM_F16)
    return launch_attn_dtype<_Float16>(group, q, hq, hkv, kc, vc, n, stride_tok, stride_head,
                                       idx, k, scale, out, lse, ws, s);
  return launch_attn_dtype<float>(group, q, hq, hkv, kc, vc, n, stride_tok, stride_head, idx, k,
                                  scale, out, lse, ws, s);
}

}  // namespace fathom
