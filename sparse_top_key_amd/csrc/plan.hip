// Read-side decision of Fathom (explainer, sections 核心方法 read side and
// 关键伪代码): reverse water-filling of each query head's bit budget.
//
// The walk "visit channels by descending importance, give each min(4, rest)
// bits" is evaluated without a sort: the channel at position j of the
// (w desc, channel asc) order receives clamp(B - 4j, 0, 4) bits, and its
// position j is its rank, i.e. the number of channels that precede it.  One
// 1024-thread block per query head: the 128x128 rank comparisons are 16 per
// thread.
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

int32_t launch_plan_fixed(const float *q, int32_t hq, int32_t r, uint8_t *plan,
                          hipStream_t s) {
  hipLaunchKernelGGL(plan_fixed_kernel, dim3(hq), dim3(kPlanThreads), 0, s, q, r, plan);
  return hip_fail(hipGetLastError(), "plan_fixed launch");
}

}  // namespace fathom
