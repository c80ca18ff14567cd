// Calibrated allocation.  The explainer's key-pseudocode section says the
// original allocates bits more finely than fill-to-cap and gives no rule; its
// intuition section ties the allocation to how much each channel's error
// moves the logit.  Here that error is measured on the layer itself:
//
//  * code_hist_kernel: per (kv head, channel) the histogram of the 4-bit codes
//    of the n keys, read from the planes (16 AND-combined plane masks per
//    32-key word, popcounted);
//  * plan_calibrated_kernel: per query head h, with E_c(t) = the summed square
//    gap between a key's 4-bit value and its t-bit cell centre (in delta^2
//    units, from the histogram; exact in fp64), the plan minimising
//    sum_c fl64(fl64(q_hc^2 delta_c^2) E_c(t_c)) under sum t_c = B, found by
//    dynamic programming over the channels in order.  One 64-lane wave per
//    head: lane l keeps the states b = l, l + 64, ... of the running minimum
//    (fp64, in registers, predecessors by lane shifts), each channel's choice
//    of t per state goes to a 128 x (B + 1) byte table in LDS, and lane 0
//    follows the choices back.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kHistThreads = 256;
constexpr int kDpThreads = 64;
constexpr int kDpHeadsPerLaunch = 64;
constexpr int kMaxBudget = kPlanes * kD;  // 512

struct DpBudgets {
  int32_t b[kDpHeadsPerLaunch];
};

// grid (hkv * kD): block (h, c) = blockIdx.x.  Rows of W words; bits of keys
// >= n are ignored (plane rows may have spare capacity).
__global__ __launch_bounds__(kHistThreads) void code_hist_kernel(const uint32_t *__restrict__ planes,
                                                                 int64_t n, int64_t W,
                                                                 uint32_t *__restrict__ hist) {
  __shared__ uint32_t s_cnt[16];
  const int tid = threadIdx.x;
  if (tid < 16) s_cnt[tid] = 0u;
  __syncthreads();
  const uint32_t *pc = planes + (int64_t)blockIdx.x * kPlanes * W;
  const int64_t nwords = (n + 31) / 32;
  uint32_t cnt[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) cnt[v] = 0u;
  // four consecutive words per thread and step (W is a multiple of 64)
  for (int64_t w0 = 4 * (int64_t)tid; w0 < nwords; w0 += 4 * kHistThreads) {
    uint4 r[kPlanes];
#pragma unroll
    for (int s = 0; s < kPlanes; ++s) r[s] = *reinterpret_cast<const uint4 *>(pc + s * W + w0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t w = w0 + e;
      const int64_t rem = n - 32 * w;  // keys of this word below n
      const uint32_t valid = rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : (1u << rem) - 1u);
      const uint32_t b3 = (&r[0].x)[e], b2 = (&r[1].x)[e], b1 = (&r[2].x)[e], b0 = (&r[3].x)[e];
      // slot 0 holds bit 3 of the code: hi pairs from bits 3, 2, lo pairs from 1, 0
      const uint32_t hp[4] = {~b3 & ~b2 & valid, ~b3 & b2 & valid, b3 & ~b2 & valid,
                              b3 & b2 & valid};
      const uint32_t lp[4] = {~b1 & ~b0, ~b1 & b0, b1 & ~b0, b1 & b0};
#pragma unroll
      for (int v = 0; v < 16; ++v) cnt[v] += (uint32_t)__popc(hp[v >> 2] & lp[v & 3]);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    uint32_t x = cnt[v];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((tid & 63) == 0) atomicAdd(&s_cnt[v], x);
  }
  __syncthreads();
  if (tid < 16) hist[(int64_t)blockIdx.x * 16 + tid] = s_cnt[tid];
}

// Whole-wave shift by one lane to the right (lane l gets lane l - 1's value;
// lane 0 gets `carry`), for fp64 values as two 32-bit DPP moves.
__device__ __forceinline__ double wave_shr1(double x, double carry) {
  const int lo = __double2loint(x), hi = __double2hiint(x);
  const int clo = __double2loint(carry), chi = __double2hiint(carry);
  const int rlo = __builtin_amdgcn_update_dpp(clo, lo, 0x138 /* wave_shr:1 */, 0xF, 0xF, false);
  const int rhi = __builtin_amdgcn_update_dpp(chi, hi, 0x138 /* wave_shr:1 */, 0xF, 0xF, false);
  return __hiloint2double(rhi, rlo);
}
// The value of lane 63, in every lane.
__device__ __forceinline__ double lane63(double x) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), 63);
  return __hiloint2double(hi, lo);
}

// One 64-lane block per query head h = h0 + blockIdx.x.  J = rounds of 64
// states per lane, enough for the largest budget of the launch (no branches
// on the budget inside the channel loop).
// A plan covers `rows` consecutive query heads from row0 = p * rows (1: per
// head; the group size: one plan per GQA group, whose weight is the fp64 sum
// in head order of the heads' squared queries, exactly q * q for one head).
template <int J>
__global__ __launch_bounds__(kDpThreads) void plan_calibrated_kernel(
    const float *__restrict__ q, int32_t group, int32_t rows, int32_t p0,
    const float *__restrict__ lo, const float *__restrict__ hi,
    const uint32_t *__restrict__ hist, DpBudgets budgets, uint8_t *__restrict__ plan) {
  __shared__ double s_cost[kD][kPlanes + 1];
  __shared__ uint8_t s_choice[kD][kMaxBudget + 1];
  __shared__ uint8_t s_plan[kD];
  const int row0 = (p0 + blockIdx.x) * rows;
  const int g = row0 / group;
  const int lane = threadIdx.x;
  const int B = budgets.b[blockIdx.x];
  // ---- per-channel costs: lane takes channels lane and lane + 64
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    const float delta = __fmul_rn(__fsub_rn(hi[g * kD + c], lo[g * kD + c]), 0.0625f);
    double sq = 0.0;
    for (int r = 0; r < rows; ++r) {
      const double qc = (double)q[(int64_t)(row0 + r) * kD + c];
      sq = __dadd_rn(sq, __dmul_rn(qc, qc));
    }
    const double qd = __dmul_rn(sq, __dmul_rn((double)delta, (double)delta));
    const uint32_t *hc = hist + ((int64_t)g * kD + c) * 16;
    uint32_t hv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) hv[v] = hc[v];
#pragma unroll
    for (int t = 0; t <= kPlanes; ++t) {
      const int m = 1 << (kPlanes - t);
      double e = 0.0;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const double off = (double)(v % m) + 0.5 - 0.5 * m;
        e = __dadd_rn(e, __dmul_rn((double)hv[v], __dmul_rn(off, off)));
      }
      s_cost[c][t] = __dmul_rn(qd, e);
    }
  }
  __syncthreads();
  // ---- F_{c+1}[b] = min_t F_c[b - t] + cost_c(t); t ascending, strict <.
  // Lane l keeps F at the states b = l + 64 j in registers (j < J).
  // F_c[b - t] reaches lane l by t shifts of one lane to the right across
  // the whole wave; lane 0 of round j takes lane 63 of round j - 1 (none for
  // j = 0: those states are negative, +inf).  No LDS round trip per channel:
  // only the choices are stored.  A depth above a state's bit count is a
  // +inf candidate, which never wins; states past B are computed but only
  // ever feed states past B.
  double f[J];
#pragma unroll
  for (int j = 0; j < J; ++j) f[j] = (lane == 0 && j == 0) ? 0.0 : INFINITY;
  double cn[kPlanes + 1];  // the next channel's costs, loaded a step ahead
#pragma unroll
  for (int t = 0; t <= kPlanes; ++t) cn[t] = s_cost[0][t];
  for (int c = 0; c < kD; ++c) {
    double ct[kPlanes + 1];
#pragma unroll
    for (int t = 0; t <= kPlanes; ++t) {
      ct[t] = cn[t];
      cn[t] = s_cost[c + 1 < kD ? c + 1 : c][t];
    }
    double sh[J], best[J];
    int bt[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      sh[j] = f[j];
      best[j] = __dadd_rn(f[j], ct[0]);  // t = 0: every state has it
      bt[j] = 0;
    }
#pragma unroll
    for (int t = 1; t <= kPlanes; ++t) {
      double nsh[J];
#pragma unroll
      for (int j = 0; j < J; ++j) nsh[j] = wave_shr1(sh[j], j > 0 ? lane63(sh[j - 1]) : INFINITY);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        sh[j] = nsh[j];
        const int b = lane + kDpThreads * j;
        const double v = t <= b ? __dadd_rn(sh[j], ct[t]) : INFINITY;
        const bool better = v < best[j];
        best[j] = better ? v : best[j];
        bt[j] = better ? t : bt[j];
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      f[j] = best[j];
      const int b = lane + kDpThreads * j;
      if (b <= B) s_choice[c][b] = (uint8_t)bt[j];
    }
  }
  __syncthreads();
  // ---- follow the choices back from F_d[B]
  if (lane == 0) {
    int b = B;
    for (int c = kD - 1; c >= 0; --c) {
      const int t = s_choice[c][b];
      s_plan[c] = (uint8_t)t;
      b -= t;
    }
  }
  __syncthreads();
  for (int r = 0; r < rows; ++r) {
    plan[(int64_t)(row0 + r) * kD + lane] = s_plan[lane];
    plan[(int64_t)(row0 + r) * kD + lane + 64] = s_plan[lane + 64];
  }
}

}  // namespace

int32_t launch_code_hist(const uint32_t *planes, int64_t n, int32_t hkv, int64_t W,
                         uint32_t *hist, hipStream_t s) {
  hipLaunchKernelGGL(code_hist_kernel, dim3((unsigned)(hkv * kD)), dim3(kHistThreads), 0, s,
                     planes, n, W, hist);
  return hip_fail(hipGetLastError(), "code_hist launch");
}

int32_t launch_plan_calibrated(const float *q, int32_t hq, int32_t hkv, const float *lo,
                               const float *hi, const uint32_t *hist,
                               const int32_t *budget_host, uint8_t *plan, bool per_group,
                               hipStream_t s) {
  const int32_t group = hq / hkv;
  const int32_t rows = per_group ? group : 1;
  const int32_t nplans = hq / rows;
  for (int32_t h0 = 0; h0 < nplans; h0 += kDpHeadsPerLaunch) {
    const int32_t cnt = std::min(kDpHeadsPerLaunch, nplans - h0);
    DpBudgets b{};
    for (int i = 0; i < cnt; ++i) b.b[i] = budget_host[h0 + i];
    int maxb = 0;
    for (int i = 0; i < cnt; ++i) maxb = std::max(maxb, b.b[i]);
    const int J = maxb / kDpThreads + 1;  // 1..9
    const dim3 grid(cnt), block(kDpThreads);
    switch (J) {
#define FATHOM_DP_CASE(K)                                                                     \
  case K:                                                                                     \
    hipLaunchKernelGGL(plan_calibrated_kernel<K>, grid, block, 0, s, q, group, rows, h0, lo, hi, \
                       hist, b, plan);                                                        \
    break;
      FATHOM_DP_CASE(1) FATHOM_DP_CASE(2) FATHOM_DP_CASE(3) FATHOM_DP_CASE(4)
      FATHOM_DP_CASE(5) FATHOM_DP_CASE(6) FATHOM_DP_CASE(7) FATHOM_DP_CASE(8)
      default: FATHOM_DP_CASE(9)
#undef FATHOM_DP_CASE
    }
  }
  return hip_fail(hipGetLastError(), "plan_calibrated launch");
}

}  // namespace fathom
