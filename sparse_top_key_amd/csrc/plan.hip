// Read-side decision of Fathom (explainer, sections 核心方法 read side and
// 关键伪代码): reverse water-filling of each query head's bit budget.
//
// The walk "visit channels by descending importance, give each min(4, rest)
// bits" is evaluated without a sort: the channel at position j of the
// (w desc, channel asc) order receives clamp(B - 4j, 0, 4) bits, and its
// position j is its rank, i.e. the number of channels that precede it.  One
// 1024-thread block per query head: the 128x128 rank comparisons are 16 per
// thread.
//
// Two variants of the allocation live here as well: the rate-distortion
// greedy (the explainer's pseudocode notes that the original allocates more
// finely than fill-to-cap; its intuition section says near-equal importances
// spread the budget) and one plan per GQA group (sharing channel importance
// across a group is listed there as a direction).
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kPlanHeadsPerLaunch = 64;
constexpr int kPlanThreads = 1024;
constexpr int kParts = kPlanThreads / kD;  // comparison slices per channel
constexpr int kPartLen = kD / kParts;

struct Budgets {
  int32_t b[kPlanHeadsPerLaunch];
};

// Rank of channel c (weight wc) in the (w desc, channel asc) order: the
// channels that precede it.  Thread (slice, c) counts those among channels
// slice*16 .. slice*16+15; the slices are summed in LDS.
__device__ __forceinline__ int rank_desc(const float *w, int c, int *part) {
  const int t = threadIdx.x, sl = t / kD;
  const float wc = w[c];
  int r = 0;
#pragma unroll
  for (int i = 0; i < kPartLen; ++i) {
    const int j = sl * kPartLen + i;
    const float wj = w[j];
    r += (wj > wc) || (wj == wc && j < c);
  }
  part[sl * kD + c] = r;
  __syncthreads();
  int rank = 0;
  if (t < kD) {
#pragma unroll
    for (int q = 0; q < kParts; ++q) rank += part[q * kD + t];
  }
  return rank;
}

// blockIdx.x = query head h0 + blockIdx.x; w_c = (q_c * q_c) * sigma2_c.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const float *__restrict__ q,
                                                            const float *__restrict__ sigma2,
                                                            int32_t group, int32_t h0,
                                                            Budgets budgets,
                                                            uint8_t *__restrict__ plan) {
  __shared__ float w[kD];
  __shared__ int part[kParts * kD];
  const int h = h0 + blockIdx.x;
  const int g = h / group;
  const int t = threadIdx.x;
  if (t < kD) {
    const float qc = q[(int64_t)h * kD + t];
    w[t] = __fmul_rn(__fmul_rn(qc, qc), sigma2[(int64_t)g * kD + t]);
  }
  __syncthreads();
  const int j = rank_desc(w, t % kD, part);
  if (t < kD) {
    const int B = budgets.b[blockIdx.x];
    plan[(int64_t)h * kD + t] = (uint8_t)min(4, max(0, B - 4 * j));
  }
}

// Fixed-width baseline: the r channels of largest |q_c| get all 4 planes.
__global__ __launch_bounds__(kPlanThreads) void plan_fixed_kernel(const float *__restrict__ q,
                                                                  int32_t r,
                                                                  uint8_t *__restrict__ plan) {
  __shared__ float w[kD];
  __shared__ int part[kParts * kD];
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  if (t < kD) w[t] = fabsf(q[(int64_t)h * kD + t]);
  __syncthreads();
  const int j = rank_desc(w, t % kD, part);
  if (t < kD) plan[(int64_t)h * kD + t] = (uint8_t)(j < r ? 4 : 0);
}

// Rate-distortion plan.  Bit t+1 of channel c (t bits already read) lowers the
// channel's error term w_c * 4^-t by an amount proportional to
// g(c, t) = w_c * 4^-t; the budget buys the B largest gains in the order
// (gain desc, c asc, t asc), which is the order (gain desc, e asc) over the
// entry index e = 4c + t.  The gains of one channel fall with t, so the bits
// bought from a channel are its top ones and t_c = #{t : rank(4c + t) < B}.
// Gains are fp64: w_c * 2^-2t is exact there, so ties are exact ties.
// Thread (half, e) ranks entry e against entries half*256 .. half*256+255.
__global__ __launch_bounds__(kPlanThreads) void plan_rd_kernel(const float *__restrict__ q,
                                                               const float *__restrict__ sigma2,
                                                               int32_t group, int32_t h0,
                                                               Budgets budgets,
                                                               uint8_t *__restrict__ plan) {
  constexpr int kEntries = kPlanes * kD;           // 512
  constexpr int kHalf = kEntries / 2;
  static_assert(kPlanThreads == 2 * kEntries, "two rank slices per entry");
  __shared__ double gain[kEntries];
  __shared__ int part[2][kEntries];
  const int h = h0 + blockIdx.x;
  const int g = h / group;
  const int t = threadIdx.x;
  if (t < kD) {
    const float qc = q[(int64_t)h * kD + t];
    const double w = (double)__fmul_rn(__fmul_rn(qc, qc), sigma2[(int64_t)g * kD + t]);
    gain[4 * t + 0] = w;
    gain[4 * t + 1] = w * 0.25;
    gain[4 * t + 2] = w * 0.0625;
    gain[4 * t + 3] = w * 0.015625;
  }
  __syncthreads();
  const int e = t % kEntries, half = t / kEntries;
  const double ge = gain[e];
  int r = 0;
#pragma unroll 8
  for (int i = 0; i < kHalf; ++i) {
    const int j = half * kHalf + i;
    const double gj = gain[j];
    r += (gj > ge) || (gj == ge && j < e);
  }
  part[half][e] = r;
  __syncthreads();
  if (t < kD) {
    const int B = budgets.b[blockIdx.x];
    int depth = 0;
#pragma unroll
    for (int k = 0; k < kPlanes; ++k) depth += (part[0][4 * t + k] + part[1][4 * t + k]) < B;
    plan[(int64_t)h * kD + t] = (uint8_t)depth;
  }
}

// One plan per GQA group: blockIdx.x = kv head g0 + blockIdx.x.  The group's
// importance of channel c is sigma2_gc * sum_j q_{gG+j,c}^2, the squares
// rounded and added in fp32 in head order, the product rounded once; the
// fill-to-cap walk spends the group's budget and every head of the group
// receives the same row.
__global__ __launch_bounds__(kPlanThreads) void plan_group_kernel(
    const float *__restrict__ q, const float *__restrict__ sigma2, int32_t group, int32_t g0,
    Budgets budgets, uint8_t *__restrict__ plan) {
  __shared__ float w[kD];
  __shared__ int part[kParts * kD];
  const int g = g0 + blockIdx.x;
  const int t = threadIdx.x;
  if (t < kD) {
    float sq = 0.0f;
    for (int j = 0; j < group; ++j) {
      const float qc = q[((int64_t)g * group + j) * kD + t];
      sq = __fadd_rn(sq, __fmul_rn(qc, qc));
    }
    w[t] = __fmul_rn(sq, sigma2[(int64_t)g * kD + t]);
  }
  __syncthreads();
  const int j = rank_desc(w, t % kD, part);
  if (t < kD) {
    const uint8_t take = (uint8_t)min(4, max(0, budgets.b[blockIdx.x] - 4 * j));
    for (int k = 0; k < group; ++k) plan[((int64_t)g * group + k) * kD + t] = take;
  }
}

}  // namespace

int32_t launch_plan(const float *q, int32_t hq, int32_t hkv, const float *sigma2,
                    const int32_t *budget_host, uint8_t *plan, hipStream_t s) {
  const int32_t group = hq / hkv;
  for (int32_t h0 = 0; h0 < hq; h0 += kPlanHeadsPerLaunch) {
    const int32_t cnt = std::min(kPlanHeadsPerLaunch, hq - h0);
    Budgets b{};
    for (int i = 0; i < cnt; ++i) b.b[i] = budget_host[h0 + i];
    hipLaunchKernelGGL(plan_kernel, dim3(cnt), dim3(kPlanThreads), 0, s, q, sigma2, group,
                       h0, b, plan);
  }
  return hip_fail(hipGetLastError(), "plan launch");
}

int32_t launch_plan_rd(const float *q, int32_t hq, int32_t hkv, const float *sigma2,
                       const int32_t *budget_host, uint8_t *plan, hipStream_t s) {
  const int32_t group = hq / hkv;
  for (int32_t h0 = 0; h0 < hq; h0 += kPlanHeadsPerLaunch) {
    const int32_t cnt = std::min(kPlanHeadsPerLaunch, hq - h0);
    Budgets b{};
    for (int i = 0; i < cnt; ++i) b.b[i] = budget_host[h0 + i];
    hipLaunchKernelGGL(plan_rd_kernel, dim3(cnt), dim3(kPlanThreads), 0, s, q, sigma2, group,
                       h0, b, plan);
  }
  return hip_fail(hipGetLastError(), "plan_rd launch");
}

int32_t launch_plan_group(const float *q, int32_t hq, int32_t hkv, const float *sigma2,
                          const int32_t *budget_host, uint8_t *plan, hipStream_t s) {
  const int32_t group = hq / hkv;
  for (int32_t g0 = 0; g0 < hkv; g0 += kPlanHeadsPerLaunch) {
    const int32_t cnt = std::min(kPlanHeadsPerLaunch, hkv - g0);
    Budgets b{};
    for (int i = 0; i < cnt; ++i) b.b[i] = budget_host[g0 + i];
    hipLaunchKernelGGL(plan_group_kernel, dim3(cnt), dim3(kPlanThreads), 0, s, q, sigma2,
                       group, g0, b, plan);
  }
  return hip_fail(hipGetLastError(), "plan_group launch");
}

int32_t launch_plan_fixed(const float *q, int32_t hq, int32_t r, uint8_t *plan,
                          hipStream_t s) {
  hipLaunchKernelGGL(plan_fixed_kernel, dim3(hq), dim3(kPlanThreads), 0, s, q, r, plan);
  return hip_fail(hipGetLastError(), "plan_fixed launch");
}

}  // namespace fathom
