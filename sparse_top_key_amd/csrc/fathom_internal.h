// Internal declarations shared by the HIP translation units of libfathom.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fathom.h"

namespace fathom {

constexpr int kD = FATHOM_HEAD_DIM;     // channels per head
constexpr int kPlanes = 4;              // 4-bit codes -> 4 bit planes
constexpr int kBlockKeys = 2048;        // keys per 64-word plane block
constexpr int kSessPerLaunch = 16;      // sessions carried in one kernarg set
constexpr int kCandCap = 8192;          // top-k candidates kept per row
constexpr int kSampleTarget = 16384;    // sampled scores per row (threshold)

// Thread-local error text behind fathom_last_error().
void set_error(const char *fmt, ...);
int32_t hip_fail(hipError_t e, const char *what);

inline int64_t plane_words(int64_t n) { return 64 * ((n + kBlockKeys - 1) / kBlockKeys); }

// ---- pack -------------------------------------------------------------------
int64_t pack_workspace_bytes(int64_t n, int32_t hkv);
int32_t launch_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                    int64_t stride_tok, int64_t stride_head, uint32_t *planes,
                    float *lo, float *hi, float *sigma2, void *ws,
                    hipStream_t s);

// ---- plan -------------------------------------------------------------------
int32_t launch_plan(const float *q, int32_t hq, int32_t hkv,
                    const float *sigma2, const int32_t *budget_host,
                    uint8_t *plan, hipStream_t s);
int32_t launch_plan_fixed(const float *q, int32_t hq, int32_t r, uint8_t *plan,
                          hipStream_t s);

// ---- scan -------------------------------------------------------------------
struct ScanSession {
  const uint32_t *planes;
  const float *lo, *hi;
  int64_t n;
  const float *q;
  const uint8_t *plan;
  const uint8_t *meta;
  float meta_scale;
  float *logits;
  int64_t ld;
};
int32_t launch_scan(const ScanSession *sess, int32_t n_sess, int32_t hkv,
                    int32_t hq, hipStream_t s);
int32_t launch_read_prefixes(const uint32_t *planes, int64_t n, int32_t hkv,
                             const uint8_t *plan, int32_t hq, uint8_t *out,
                             hipStream_t s);

// ---- top-k ------------------------------------------------------------------
struct TopkSession {
  const float *scores;  // first input row of the session
  int64_t n, ld;
  int32_t *idx;
  float *vals;
};
int64_t topk_workspace_bytes(int32_t out_rows);
int32_t launch_topk(const TopkSession *sess, int32_t n_sess, int32_t rows_per_sess,
                    int32_t group, int32_t k, void *ws, hipStream_t s);

// ---- probe ------------------------------------------------------------------
int32_t launch_probe_read(const void *src, int64_t bytes, uint32_t *out,
                          int32_t blocks, hipStream_t s);

}  // namespace fathom
