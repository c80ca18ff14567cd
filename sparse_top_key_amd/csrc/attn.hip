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
// one index row; each wave owns 64 of them and the block merges its waves'
// (m, l, o[128]) into one partial per query head of the row.  The wave's V
// rows are read row by row, one coalesced 256-byte row per instruction (lane
// l holds channels 2l, 2l+1), the first batch (64 fp16 rows, 32 fp32 rows)
// issued before the K rows so that the two gathers' latencies overlap; lane j
// scores entry j from its own K row (16-byte loads, q broadcast from LDS).
// attn_combine_kernel merges a head's block partials by their maxima.
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
// Block b writes the merged partial of its 256 entries for each head:
// part[((r * nparts + b) * GH + j) * kPart + ...], nparts = gridDim.x.
template <typename T, int GH>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(
    const float *__restrict__ q, int32_t heads_per_kv, const T *__restrict__ kc,
    const T *__restrict__ vc, int64_t n, int64_t stride_tok, int64_t stride_head,
    const int32_t *__restrict__ idx, int32_t k, float scale, float *__restrict__ part) {
  using E = Elem<T>;
  using Pair = typename E::Pair;
  constexpr int kVecs = kD / E::kPerVec;       // 16-byte vectors per K row
  constexpr int kKChunk = 16;                   // K vectors in flight per lane
  constexpr int kVBatch = 256 / sizeof(Pair);   // V rows in flight per wave

  __shared__ float s_q[GH][kD];
  __shared__ float s_ml[kAttnWaves][GH][2];     // per wave: max, sum of weights
  __shared__ float s_o[kAttnWaves][GH][kD];     // per wave: weighted V sums
  const int r = blockIdx.y;
  const int h0 = r * GH;
  const int g = h0 / heads_per_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < GH * kD; e += kAttnThreads) s_q[e / kD][e % kD] = q[(int64_t)h0 * kD + e];

  const int j = blockIdx.x * kAttnBlockKeys + wave * 64 + lane;
  int key = -1;
  if (j < k) {
    const int v = idx[(int64_t)r * k + j];
    key = (v >= 0 && v < n) ? v : -1;  // padding and out-of-range entries are skipped
  }
  const int64_t head_off = (int64_t)g * stride_head;
  const bool any = __ballot(key >= 0) != 0ull;

  // ---- first batch of V rows, issued before the K rows: lane l holds
  // channels 2l, 2l+1; a skipped entry reads row 0 with weight 0 -------------
  Pair vr[kVBatch];
  auto load_v = [&](int j0) {
#pragma unroll
    for (int jj = 0; jj < kVBatch; ++jj) {
      const int kj = __builtin_amdgcn_readlane(key, j0 + jj);
      const int64_t row = kj >= 0 ? kj : 0;
      vr[jj] = *reinterpret_cast<const Pair *>(vc + row * stride_tok + head_off + 2 * lane);
    }
  };
  if (any) load_v(0);
  __syncthreads();  // s_q

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

  float m[GH], p[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const float sc = key >= 0 ? __fmul_rn(scale, dot[h]) : -INFINITY;
    m[h] = wave_max(sc);
    p[h] = key >= 0 ? expf(__fsub_rn(sc, m[h])) : 0.0f;
    const float l = wave_sum(p[h]);
    if (lane == 0) {
      s_ml[wave][h][0] = m[h];
      s_ml[wave][h][1] = l;
    }
  }

  // ---- o = sum_j p_j V_j over the wave's entries, in entry order -----------
  float o0[GH], o1[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) o0[h] = o1[h] = 0.0f;
  if (any) {
#pragma unroll
    for (int j0 = 0; j0 < 64; j0 += kVBatch) {
      if (j0 > 0) load_v(j0);
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
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    s_o[wave][h][2 * lane] = o0[h];
    s_o[wave][h][2 * lane + 1] = o1[h];
  }
  __syncthreads();

  // ---- merge the block's waves in wave order: thread (h, c) ----------------
  for (int e = tid; e < GH * kD; e += kAttnThreads) {
    const int h = e / kD, c = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = s_ml[w][h][0];
        const float sc = mw == -INFINITY ? 0.0f : expf(__fsub_rn(mw, M));
        L = fmaf(sc, s_ml[w][h][1], L);
        o = fmaf(sc, s_o[w][h][c], o);
      }
    }
    float *dst = part + ((int64_t)(r * gridDim.x + blockIdx.x) * GH + h) * kPart;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
    dst[2 + c] = o;
  }
}

// One block of kD threads per query head h (idx row h / GH, head h % GH):
// the block partials of the head, merged by their maxima in block order.
// Loads are issued kUnroll at a time so their latencies overlap.
template <int GH>
__global__ __launch_bounds__(kD) void attn_combine_kernel(const float *__restrict__ part,
                                                          int32_t nparts,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
  constexpr int kUnroll = 8;
  const int h = blockIdx.x, c = threadIdx.x;
  const int r = h / GH, hh = h % GH;
  const float *base = part + ((int64_t)r * nparts * GH + hh) * kPart;
  const int64_t step = (int64_t)GH * kPart;
  float M = -INFINITY;
  for (int i0 = 0; i0 < nparts; i0 += kUnroll) {
    float mv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      mv[u] = i0 + u < nparts ? base[(i0 + u) * step] : -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) M = fmaxf(M, mv[u]);
  }
  float L = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
    for (int i0 = 0; i0 < nparts; i0 += kUnroll) {
      float mv[kUnroll], lv[kUnroll], ov[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bool in = i0 + u < nparts;
        const float *pp = base + (in ? (i0 + u) * step : 0);
        mv[u] = in ? pp[0] : -INFINITY;
        lv[u] = pp[1];
        ov[u] = pp[2 + c];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (mv[u] == -INFINITY) continue;
        const float w = expf(__fsub_rn(mv[u], M));
        L = fmaf(w, lv[u], L);
        o = fmaf(w, ov[u], o);
      }
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
  const int32_t nparts = (k + kAttnBlockKeys - 1) / kAttnBlockKeys;
  float *part = static_cast<float *>(ws);
  if (nparts > 0) {
    const dim3 grid(nparts, rows);
    hipLaunchKernelGGL((attn_partial_kernel<T, GH>), grid, dim3(kAttnThreads), 0, s, q, hq / hkv,
                       static_cast<const T *>(kc), static_cast<const T *>(vc), n, stride_tok,
                       stride_head, idx, k, scale, part);
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
  return (int64_t)hq * ((k + kAttnBlockKeys - 1) / kAttnBlockKeys) * kPart *
         (int64_t)sizeof(float);
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
