// Exported C ABI of libfathom (declared in include/fathom.h): argument
// validation on the host, then kernel launches on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fathom_internal.h"

namespace fathom {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int32_t hip_fail(hipError_t e, const char *what) {
  if (e == hipSuccess) return FATHOM_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return FATHOM_ERR_HIP;
}

}  // namespace fathom

using namespace fathom;

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) {               \
      set_error(__VA_ARGS__);    \
      return (code);             \
    }                            \
  } while (0)

static hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

static int32_t check_d(int32_t d) {
  REQUIRE(d > 0, FATHOM_ERR_INVALID_ARG, "d must be positive (got %d)", d);
  REQUIRE(d == kD, FATHOM_ERR_UNSUPPORTED, "only d == %d is implemented (got %d)", kD, d);
  return FATHOM_OK;
}

static int32_t check_heads(int32_t hq, int32_t hkv) {
  REQUIRE(hkv >= 1 && hq >= 1, FATHOM_ERR_INVALID_ARG, "hq and hkv must be >= 1");
  REQUIRE(hq % hkv == 0, FATHOM_ERR_INVALID_ARG, "hq (%d) must be a multiple of hkv (%d)",
          hq, hkv);
  return FATHOM_OK;
}

extern "C" {

int32_t fathom_abi_version(void) { return FATHOM_ABI_VERSION; }

const char *fathom_last_error(void) { return g_err; }

int64_t fathom_plane_words(int64_t n) { return n < 0 ? 0 : plane_words(n); }

int64_t fathom_planes_bytes(int64_t n, int32_t hkv, int32_t d) {
  if (n < 0 || hkv < 1 || d < 1) return 0;
  return (int64_t)hkv * d * kPlanes * plane_words(n) * (int64_t)sizeof(uint32_t);
}

int64_t fathom_pack_workspace_bytes(int64_t n, int32_t hkv, int32_t d) {
  if (n < 1 || hkv < 1 || d != kD) return 0;
  return pack_workspace_bytes(n, hkv);
}

int64_t fathom_topk_workspace_bytes(int32_t out_rows, int32_t k) {
  if (out_rows < 1 || k < 1 || k > FATHOM_MAX_K) return 0;
  return topk_workspace_bytes(out_rows);
}

int32_t fathom_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv, int32_t d,
                    int64_t stride_tok, int64_t stride_head, uint32_t *planes, float *lo,
                    float *hi, float *sigma2, void *ws, int64_t ws_bytes, void *stream) {
  REQUIRE(keys && planes && lo && hi && sigma2, FATHOM_ERR_INVALID_ARG,
          "fathom_pack: null pointer");
  REQUIRE(dtype == FATHOM_F16 || dtype == FATHOM_F32, FATHOM_ERR_INVALID_ARG,
          "fathom_pack: dtype must be FATHOM_F16 or FATHOM_F32 (got %d)", dtype);
  REQUIRE(n >= 1 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_pack: n must be in [1, 2^31] (got %lld)", (long long)n);
  REQUIRE(hkv >= 1, FATHOM_ERR_INVALID_ARG, "fathom_pack: hkv must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(stride_tok >= 0 && stride_head >= 0, FATHOM_ERR_INVALID_ARG,
          "fathom_pack: strides must be non-negative");
  const int64_t need = pack_workspace_bytes(n, hkv);
  REQUIRE(ws && ws_bytes >= need, FATHOM_ERR_WORKSPACE,
          "fathom_pack: workspace of %lld bytes needed (got %lld)", (long long)need,
          (long long)ws_bytes);
  return launch_pack(keys, dtype, n, hkv, stride_tok, stride_head, planes, lo, hi, 0, sigma2,
                     ws, as_stream(stream));
}

int64_t fathom_range_blocks(int64_t n) {
  return n < 0 ? 0 : (n + kBlockKeys - 1) / kBlockKeys;
}

int64_t fathom_pack_blocked_workspace_bytes(int64_t n, int32_t hkv, int32_t d) {
  if (n < 1 || hkv < 1 || d != kD) return 0;
  return pack_blocked_workspace_bytes(n, hkv);
}

// Range rows of per-block layers: at least the blocks of n keys, at most 2^20
// (the blocks of 2^31 keys).
static int32_t check_range_stride(int64_t rs, int64_t n, const char *who) {
  REQUIRE(rs >= fathom_range_blocks(n) && rs >= 1 && rs <= ((int64_t)1 << 20),
          FATHOM_ERR_INVALID_ARG, "%s: range_stride (%lld) must be in [%lld, 2^20]", who,
          (long long)rs, (long long)std::max<int64_t>(1, fathom_range_blocks(n)));
  return FATHOM_OK;
}

int32_t fathom_pack_blocked(const void *keys, int32_t dtype, int64_t n, int32_t hkv, int32_t d,
                            int64_t stride_tok, int64_t stride_head, uint32_t *planes,
                            float *lo, float *hi, int64_t range_stride, float *sigma2,
                            void *ws, int64_t ws_bytes, void *stream) {
  REQUIRE(keys && planes && lo && hi && sigma2, FATHOM_ERR_INVALID_ARG,
          "fathom_pack_blocked: null pointer");
  REQUIRE(dtype == FATHOM_F16 || dtype == FATHOM_F32, FATHOM_ERR_INVALID_ARG,
          "fathom_pack_blocked: dtype must be FATHOM_F16 or FATHOM_F32 (got %d)", dtype);
  REQUIRE(n >= 1 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_pack_blocked: n must be in [1, 2^31] (got %lld)", (long long)n);
  REQUIRE(hkv >= 1, FATHOM_ERR_INVALID_ARG, "fathom_pack_blocked: hkv must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(stride_tok >= 0 && stride_head >= 0, FATHOM_ERR_INVALID_ARG,
          "fathom_pack_blocked: strides must be non-negative");
  if (int32_t rc = check_range_stride(range_stride, n, "fathom_pack_blocked")) return rc;
  const int64_t need = pack_blocked_workspace_bytes(n, hkv);
  REQUIRE(ws && ws_bytes >= need, FATHOM_ERR_WORKSPACE,
          "fathom_pack_blocked: workspace of %lld bytes needed (got %lld)", (long long)need,
          (long long)ws_bytes);
  return launch_pack(keys, dtype, n, hkv, stride_tok, stride_head, planes, lo, hi,
                     range_stride, sigma2, ws, as_stream(stream));
}

int32_t fathom_plan(const float *q, int32_t hq, int32_t hkv, int32_t d,
                    const float *sigma2, const int32_t *budget_bits, uint8_t *plan,
                    void *stream) {
  REQUIRE(q && sigma2 && budget_bits && plan, FATHOM_ERR_INVALID_ARG,
          "fathom_plan: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  for (int32_t h = 0; h < hq; ++h)
    REQUIRE(budget_bits[h] >= 0 && budget_bits[h] <= 4 * d, FATHOM_ERR_INVALID_ARG,
            "fathom_plan: budget_bits[%d] = %d outside [0, %d]", h, budget_bits[h], 4 * d);
  return launch_plan(q, hq, hkv, sigma2, budget_bits, plan, as_stream(stream));
}

int32_t fathom_plan_rd(const float *q, int32_t hq, int32_t hkv, int32_t d,
                       const float *sigma2, const int32_t *budget_bits, uint8_t *plan,
                       void *stream) {
  REQUIRE(q && sigma2 && budget_bits && plan, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_rd: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  for (int32_t h = 0; h < hq; ++h)
    REQUIRE(budget_bits[h] >= 0 && budget_bits[h] <= 4 * d, FATHOM_ERR_INVALID_ARG,
            "fathom_plan_rd: budget_bits[%d] = %d outside [0, %d]", h, budget_bits[h], 4 * d);
  return launch_plan_rd(q, hq, hkv, sigma2, budget_bits, plan, as_stream(stream));
}

int32_t fathom_plan_group(const float *q, int32_t hq, int32_t hkv, int32_t d,
                          const float *sigma2, const int32_t *budget_bits, uint8_t *plan,
                          void *stream) {
  REQUIRE(q && sigma2 && budget_bits && plan, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_group: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  for (int32_t g = 0; g < hkv; ++g)
    REQUIRE(budget_bits[g] >= 0 && budget_bits[g] <= 4 * d, FATHOM_ERR_INVALID_ARG,
            "fathom_plan_group: budget_bits[%d] = %d outside [0, %d]", g, budget_bits[g],
            4 * d);
  return launch_plan_group(q, hq, hkv, sigma2, budget_bits, plan, as_stream(stream));
}

int32_t fathom_append(const void *keys, int32_t dtype, int64_t m, int32_t hkv, int32_t d,
                      int64_t stride_tok, int64_t stride_head, int64_t n_old,
                      uint32_t *planes, int64_t plane_words_, const float *lo,
                      const float *hi, uint32_t *clamped, void *stream) {
  REQUIRE(planes && lo && hi && (keys || m == 0), FATHOM_ERR_INVALID_ARG,
          "fathom_append: null pointer");
  REQUIRE(dtype == FATHOM_F16 || dtype == FATHOM_F32, FATHOM_ERR_INVALID_ARG,
          "fathom_append: dtype must be FATHOM_F16 or FATHOM_F32 (got %d)", dtype);
  REQUIRE(hkv >= 1, FATHOM_ERR_INVALID_ARG, "fathom_append: hkv must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(m >= 0 && n_old >= 0 && n_old + m <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_append: need m >= 0, n_old >= 0, n_old + m <= 2^31");
  REQUIRE(stride_tok >= 0 && stride_head >= 0, FATHOM_ERR_INVALID_ARG,
          "fathom_append: strides must be non-negative");
  REQUIRE(plane_words_ >= plane_words(n_old + m) && plane_words_ % 64 == 0 &&
              plane_words_ <= ((int64_t)1 << 26),
          FATHOM_ERR_INVALID_ARG,
          "fathom_append: plane_words (%lld) must be a multiple of 64 in [%lld, 2^26]",
          (long long)plane_words_, (long long)plane_words(n_old + m));
  if (m == 0) return FATHOM_OK;
  return launch_append(keys, dtype, m, hkv, stride_tok, stride_head, n_old, planes,
                       plane_words_, const_cast<float *>(lo), const_cast<float *>(hi), 0,
                       clamped, as_stream(stream));
}

int32_t fathom_append_blocked(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                              int32_t d, int64_t stride_tok, int64_t stride_head,
                              int64_t n_old, uint32_t *planes, int64_t plane_words_,
                              float *lo, float *hi, int64_t range_stride, uint32_t *clamped,
                              void *stream) {
  REQUIRE(planes && lo && hi && (keys || m == 0), FATHOM_ERR_INVALID_ARG,
          "fathom_append_blocked: null pointer");
  REQUIRE(dtype == FATHOM_F16 || dtype == FATHOM_F32, FATHOM_ERR_INVALID_ARG,
          "fathom_append_blocked: dtype must be FATHOM_F16 or FATHOM_F32 (got %d)", dtype);
  REQUIRE(hkv >= 1, FATHOM_ERR_INVALID_ARG, "fathom_append_blocked: hkv must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(m >= 0 && n_old >= 0 && n_old + m <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_append_blocked: need m >= 0, n_old >= 0, n_old + m <= 2^31");
  REQUIRE(stride_tok >= 0 && stride_head >= 0, FATHOM_ERR_INVALID_ARG,
          "fathom_append_blocked: strides must be non-negative");
  REQUIRE(plane_words_ >= plane_words(n_old + m) && plane_words_ % 64 == 0 &&
              plane_words_ <= ((int64_t)1 << 26),
          FATHOM_ERR_INVALID_ARG,
          "fathom_append_blocked: plane_words (%lld) must be a multiple of 64 in [%lld, 2^26]",
          (long long)plane_words_, (long long)plane_words(n_old + m));
  if (int32_t rc = check_range_stride(range_stride, n_old + m, "fathom_append_blocked"))
    return rc;
  if (m == 0) return FATHOM_OK;
  return launch_append(keys, dtype, m, hkv, stride_tok, stride_head, n_old, planes,
                       plane_words_, lo, hi, range_stride, clamped, as_stream(stream));
}

int64_t fathom_attention_workspace_bytes(int32_t hq, int32_t k) {
  if (hq < 1 || k < 0 || k > FATHOM_MAX_ATTN_K) return 0;
  return attn_workspace_bytes(hq, k);
}

int32_t fathom_sparse_attention(const float *q, int32_t hq, int32_t hkv, int32_t d,
                                const void *k_cache, const void *v_cache, int32_t dtype,
                                int64_t n, int64_t stride_tok, int64_t stride_head,
                                const int32_t *idx, int32_t group, int32_t k, float scale,
                                float *out, float *lse, void *ws, int64_t ws_bytes,
                                void *stream) {
  REQUIRE(q && out && lse && (idx || k == 0), FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(dtype == FATHOM_F16 || dtype == FATHOM_F32, FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: dtype must be FATHOM_F16 or FATHOM_F32 (got %d)", dtype);
  REQUIRE(n >= 0 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: n must be in [0, 2^31] (got %lld)", (long long)n);
  REQUIRE(n == 0 || (k_cache && v_cache), FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: null K or V cache");
  REQUIRE(k >= 0 && k <= FATHOM_MAX_ATTN_K, FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: k must be in [0, %d] (got %d)", FATHOM_MAX_ATTN_K, k);
  REQUIRE(group >= 1 && (hq / hkv) % group == 0, FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: group (%d) must divide hq / hkv (%d)", group, hq / hkv);
  REQUIRE(group == 1 || group == 2 || group == 4 || group == 8, FATHOM_ERR_UNSUPPORTED,
          "fathom_sparse_attention: group must be 1, 2, 4 or 8 (got %d)", group);
  REQUIRE(hq / group <= 65535, FATHOM_ERR_UNSUPPORTED,
          "fathom_sparse_attention: at most 65535 index rows (got %d)", hq / group);
  REQUIRE(std::isfinite(scale), FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: scale must be finite");
  REQUIRE(stride_tok >= 0 && stride_head >= 0, FATHOM_ERR_INVALID_ARG,
          "fathom_sparse_attention: strides must be non-negative");
  const int64_t vec = dtype == FATHOM_F16 ? 8 : 4;  // elements per 16 bytes
  REQUIRE(stride_tok % vec == 0 && stride_head % vec == 0 &&
              (reinterpret_cast<uintptr_t>(k_cache) & 15) == 0 &&
              (reinterpret_cast<uintptr_t>(v_cache) & 15) == 0,
          FATHOM_ERR_UNSUPPORTED,
          "fathom_sparse_attention: K and V rows must start on 16-byte boundaries "
          "(16-byte aligned caches, strides multiples of %lld elements)", (long long)vec);
  const int64_t need = attn_workspace_bytes(hq, k);
  REQUIRE(k == 0 || (ws && ws_bytes >= need), FATHOM_ERR_WORKSPACE,
          "fathom_sparse_attention: workspace of %lld bytes needed (got %lld)",
          (long long)need, (long long)ws_bytes);
  return launch_attention(q, hq, hkv, k_cache, v_cache, dtype, n, stride_tok, stride_head, idx,
                          group, k, scale, out, lse, ws, as_stream(stream));
}

int32_t fathom_code_hist(const uint32_t *planes, int64_t n, int32_t hkv, int32_t d,
                         int64_t plane_words_, uint32_t *hist, void *stream) {
  REQUIRE(planes && hist, FATHOM_ERR_INVALID_ARG, "fathom_code_hist: null pointer");
  REQUIRE(hkv >= 1, FATHOM_ERR_INVALID_ARG, "fathom_code_hist: hkv must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(n >= 0 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_code_hist: n must be in [0, 2^31] (got %lld)", (long long)n);
  const int64_t W = plane_words_ == 0 ? plane_words(n) : plane_words_;
  REQUIRE(W >= plane_words(n) && W % 64 == 0 && W <= ((int64_t)1 << 26),
          FATHOM_ERR_INVALID_ARG,
          "fathom_code_hist: plane_words (%lld) must be 0 or a multiple of 64 in [%lld, 2^26]",
          (long long)plane_words_, (long long)plane_words(n));
  REQUIRE((reinterpret_cast<uintptr_t>(planes) & 15) == 0, FATHOM_ERR_UNSUPPORTED,
          "fathom_code_hist: planes must be 16-byte aligned");
  return launch_code_hist(planes, n, hkv, W, hist, as_stream(stream));
}

int32_t fathom_plan_calibrated(const float *q, int32_t hq, int32_t hkv, int32_t d,
                               const float *lo, const float *hi, const uint32_t *hist,
                               const int32_t *budget_bits, uint8_t *plan, void *stream) {
  REQUIRE(q && lo && hi && hist && budget_bits && plan, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_calibrated: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  for (int32_t h = 0; h < hq; ++h)
    REQUIRE(budget_bits[h] >= 0 && budget_bits[h] <= 4 * d, FATHOM_ERR_INVALID_ARG,
            "fathom_plan_calibrated: budget_bits[%d] = %d outside [0, %d]", h, budget_bits[h],
            4 * d);
  return launch_plan_calibrated(q, hq, hkv, lo, hi, hist, budget_bits, plan, false,
                                as_stream(stream));
}

int32_t fathom_plan_calibrated_group(const float *q, int32_t hq, int32_t hkv, int32_t d,
                                     const float *lo, const float *hi, const uint32_t *hist,
                                     const int32_t *budget_bits, uint8_t *plan, void *stream) {
  REQUIRE(q && lo && hi && hist && budget_bits && plan, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_calibrated_group: null pointer");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  for (int32_t g = 0; g < hkv; ++g)
    REQUIRE(budget_bits[g] >= 0 && budget_bits[g] <= 4 * d, FATHOM_ERR_INVALID_ARG,
            "fathom_plan_calibrated_group: budget_bits[%d] = %d outside [0, %d]", g,
            budget_bits[g], 4 * d);
  return launch_plan_calibrated(q, hq, hkv, lo, hi, hist, budget_bits, plan, true,
                                as_stream(stream));
}

int32_t fathom_plan_fixed(const float *q, int32_t hq, int32_t d, int32_t r, uint8_t *plan,
                          void *stream) {
  REQUIRE(q && plan, FATHOM_ERR_INVALID_ARG, "fathom_plan_fixed: null pointer");
  REQUIRE(hq >= 1, FATHOM_ERR_INVALID_ARG, "fathom_plan_fixed: hq must be >= 1");
  if (int32_t rc = check_d(d)) return rc;
  REQUIRE(r >= 0 && r <= d, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_fixed: r = %d outside [0, %d]", r, d);
  return launch_plan_fixed(q, hq, r, plan, as_stream(stream));
}

// Plane row length of a session: 0 (fathom_plane_words(n)) or a capacity of
// at least that many words, in whole 2048-key blocks.
static int32_t check_plane_words(const fathom_session &s, const char *who) {
  REQUIRE(s.plane_words == 0 ||
              (s.plane_words >= plane_words(s.n) && s.plane_words % 64 == 0 &&
               s.plane_words <= ((int64_t)1 << 26)),
          FATHOM_ERR_INVALID_ARG,
          "%s: plane_words (%lld) must be 0 or a multiple of 64 in [%lld, 2^26]", who,
          (long long)s.plane_words, (long long)plane_words(s.n));
  return FATHOM_OK;
}

static int32_t check_scan_session(const fathom_session &s, int32_t hq, const char *who) {
  REQUIRE(s.n >= 0 && s.n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "%s: n must be in [0, 2^31] (got %lld)", who, (long long)s.n);
  if (int32_t rc = check_plane_words(s, who)) return rc;
  if (s.n == 0) return FATHOM_OK;
  REQUIRE(s.planes && s.lo && s.hi && s.q && s.plan && s.logits, FATHOM_ERR_INVALID_ARG,
          "%s: null pointer", who);
  REQUIRE(s.ld_logits >= s.n, FATHOM_ERR_INVALID_ARG, "%s: ld_logits (%lld) < n (%lld)",
          who, (long long)s.ld_logits, (long long)s.n);
  (void)hq;
  return FATHOM_OK;
}

static ScanSession to_scan(const fathom_session &s) {
  ScanSession o{};  // fused-path fields stay null
  o.planes = s.planes;
  o.lo = s.lo;
  o.hi = s.hi;
  o.n = s.n;
  o.q = s.q;
  o.plan = s.plan;
  o.meta = s.meta;
  o.meta_scale = s.meta_scale;
  o.logits = s.logits;
  o.ld = s.ld_logits;
  o.W = s.plane_words;
  return o;
}

int32_t fathom_scan(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
                    int32_t hkv, int32_t d, const float *q, const uint8_t *plan, int32_t hq,
                    const uint8_t *meta, float meta_scale, float *logits, int64_t ld_logits,
                    void *stream) {
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.meta = meta;
  s.meta_scale = meta_scale;
  s.logits = logits;
  s.ld_logits = ld_logits;
  if (int32_t rc = check_scan_session(s, hq, "fathom_scan")) return rc;
  if (n == 0) return FATHOM_OK;
  ScanSession ss = to_scan(s);
  return launch_scan(&ss, 1, hkv, hq, as_stream(stream));
}

int32_t fathom_scan_meta4(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
                          int32_t hkv, int32_t d, const float *q, const uint8_t *plan,
                          int32_t hq, const uint8_t *meta4, float meta_scale, float *logits,
                          int64_t ld_logits, void *stream) {
  REQUIRE(meta4 || n == 0, FATHOM_ERR_INVALID_ARG, "fathom_scan_meta4: null side stream");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.meta = meta4;
  s.meta_scale = meta_scale;
  s.logits = logits;
  s.ld_logits = ld_logits;
  if (int32_t rc = check_scan_session(s, hq, "fathom_scan_meta4")) return rc;
  if (n == 0) return FATHOM_OK;
  ScanSession ss = to_scan(s);
  ss.meta_bits = 4;
  return launch_scan(&ss, 1, hkv, hq, as_stream(stream));
}

int32_t fathom_scan_blocked(const uint32_t *planes, const float *lo, const float *hi,
                            int64_t range_stride, int64_t n, int32_t hkv, int32_t d,
                            const float *q, const uint8_t *plan, int32_t hq,
                            int64_t plane_words_, float *logits, int64_t ld_logits,
                            void *stream) {
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.logits = logits;
  s.ld_logits = ld_logits;
  s.plane_words = plane_words_;
  if (int32_t rc = check_scan_session(s, hq, "fathom_scan_blocked")) return rc;
  if (int32_t rc = check_range_stride(range_stride, n, "fathom_scan_blocked")) return rc;
  if (n == 0) return FATHOM_OK;
  ScanSession ss = to_scan(s);
  ss.rs = range_stride;
  return launch_scan(&ss, 1, hkv, hq, as_stream(stream));
}

int32_t fathom_scan_batched(const fathom_session *sessions, int32_t n_sessions, int32_t hkv,
                            int32_t d, int32_t hq, void *stream) {
  REQUIRE(sessions, FATHOM_ERR_INVALID_ARG, "fathom_scan_batched: null sessions");
  REQUIRE(n_sessions >= 1 && n_sessions <= FATHOM_MAX_SESSIONS, FATHOM_ERR_INVALID_ARG,
          "fathom_scan_batched: n_sessions must be in [1, %d]", FATHOM_MAX_SESSIONS);
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  ScanSession ss[FATHOM_MAX_SESSIONS];
  int32_t m = 0;
  for (int32_t i = 0; i < n_sessions; ++i) {
    if (int32_t rc = check_scan_session(sessions[i], hq, "fathom_scan_batched")) return rc;
    if (sessions[i].n > 0) ss[m++] = to_scan(sessions[i]);
  }
  if (m == 0) return FATHOM_OK;
  return launch_scan(ss, m, hkv, hq, as_stream(stream));
}

static int32_t check_topk_common(int32_t rows, int32_t group, int32_t k, const char *who) {
  REQUIRE(rows >= 1 && group >= 1 && rows % group == 0, FATHOM_ERR_INVALID_ARG,
          "%s: rows (%d) must be a positive multiple of group (%d)", who, rows, group);
  REQUIRE(k >= 1 && k <= FATHOM_MAX_K, FATHOM_ERR_INVALID_ARG,
          "%s: k = %d outside [1, %d]", who, k, FATHOM_MAX_K);
  return FATHOM_OK;
}

int32_t fathom_topk(const float *scores, int32_t rows, int64_t n, int64_t ld, int32_t group,
                    int32_t k, int32_t *idx, float *vals, void *ws, int64_t ws_bytes,
                    void *stream) {
  if (int32_t rc = check_topk_common(rows, group, k, "fathom_topk")) return rc;
  REQUIRE(idx && vals, FATHOM_ERR_INVALID_ARG, "fathom_topk: null output");
  REQUIRE(n >= 0 && n < ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_topk: n must be in [0, 2^31)");
  REQUIRE(n == 0 || scores, FATHOM_ERR_INVALID_ARG, "fathom_topk: null scores");
  REQUIRE(ld >= n, FATHOM_ERR_INVALID_ARG, "fathom_topk: ld < n");
  const int64_t need = topk_workspace_bytes(rows / group);
  REQUIRE(ws && ws_bytes >= need, FATHOM_ERR_WORKSPACE,
          "fathom_topk: workspace of %lld bytes needed (got %lld)", (long long)need,
          (long long)ws_bytes);
  TopkSession t{scores, nullptr, n, ld, idx, vals, n};
  const TopkWs w = topk_ws_carve(ws, rows / group, rows / group);
  return launch_topk(&t, 1, rows / group, group, k, w, as_stream(stream));
}

int32_t fathom_topk_noalloc(const float *scores, int32_t rows, int64_t n, int64_t ld,
                            int32_t group, int32_t k, int32_t *idx, float *vals,
                            void *stream) {
  if (int32_t rc = check_topk_common(rows, group, k, "fathom_topk_noalloc")) return rc;
  REQUIRE(idx && vals, FATHOM_ERR_INVALID_ARG, "fathom_topk_noalloc: null output");
  REQUIRE(n >= 0 && n < ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_topk_noalloc: n must be in [0, 2^31)");
  REQUIRE(n == 0 || scores, FATHOM_ERR_INVALID_ARG, "fathom_topk_noalloc: null scores");
  REQUIRE(ld >= n, FATHOM_ERR_INVALID_ARG, "fathom_topk_noalloc: ld < n");
  const int32_t out_rows = rows / group;
  REQUIRE(out_rows <= FATHOM_NOALLOC_MAX_ROWS, FATHOM_ERR_WORKSPACE,
          "fathom_topk_noalloc: %d output rows exceed the static scratch's %d",
          out_rows, FATHOM_NOALLOC_MAX_ROWS);
  const int64_t need = topk_workspace_bytes(out_rows);
  REQUIRE(need <= noalloc_scratch_bytes(), FATHOM_ERR_WORKSPACE,
          "fathom_topk_noalloc: %lld bytes of scratch needed, %lld held", (long long)need,
          (long long)noalloc_scratch_bytes());
  void *ws = nullptr;
  if (int32_t rc = noalloc_scratch(&ws)) return rc;
  TopkSession t{scores, nullptr, n, ld, idx, vals, n};
  const TopkWs w = topk_ws_carve(ws, out_rows, out_rows);
  return launch_topk(&t, 1, out_rows, group, k, w, as_stream(stream));
}

int32_t fathom_topk_batched(const fathom_session *sessions, int32_t n_sessions, int32_t hq,
                            int32_t group, int32_t k, void *ws, int64_t ws_bytes,
                            void *stream) {
  REQUIRE(sessions, FATHOM_ERR_INVALID_ARG, "fathom_topk_batched: null sessions");
  REQUIRE(n_sessions >= 1 && n_sessions <= FATHOM_MAX_SESSIONS, FATHOM_ERR_INVALID_ARG,
          "fathom_topk_batched: n_sessions must be in [1, %d]", FATHOM_MAX_SESSIONS);
  if (int32_t rc = check_topk_common(hq, group, k, "fathom_topk_batched")) return rc;
  TopkSession ts[FATHOM_MAX_SESSIONS];
  for (int32_t i = 0; i < n_sessions; ++i) {
    const fathom_session &s = sessions[i];
    REQUIRE(s.idx && s.vals, FATHOM_ERR_INVALID_ARG, "fathom_topk_batched: null output");
    REQUIRE(s.n >= 0 && s.n < ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
            "fathom_topk_batched: n must be in [0, 2^31)");
    REQUIRE(s.n == 0 || s.logits, FATHOM_ERR_INVALID_ARG, "fathom_topk_batched: null logits");
    REQUIRE(s.ld_logits >= s.n, FATHOM_ERR_INVALID_ARG, "fathom_topk_batched: ld < n");
    ts[i] = TopkSession{s.logits, nullptr, s.n, s.ld_logits, s.idx, s.vals, s.n};
  }
  const int32_t out_rows = n_sessions * (hq / group);
  const int64_t need = topk_workspace_bytes(out_rows);
  REQUIRE(ws && ws_bytes >= need, FATHOM_ERR_WORKSPACE,
          "fathom_topk_batched: workspace of %lld bytes needed (got %lld)", (long long)need,
          (long long)ws_bytes);
  const TopkWs w = topk_ws_carve(ws, out_rows, out_rows);
  return launch_topk(ts, n_sessions, hq / group, group, k, w, as_stream(stream));
}

int64_t fathom_scan_topk_workspace_bytes(const int64_t *n_host, int32_t n_sessions,
                                         int32_t hkv, int32_t hq, int32_t group, int32_t k) {
  if (!n_host || n_sessions < 1 || n_sessions > FATHOM_MAX_SESSIONS || hkv < 1 || hq < 1 ||
      hq % hkv != 0 || group < 1 || hq % group != 0 || k < 1 || k > FATHOM_MAX_K)
    return 0;
  for (int32_t i = 0; i < n_sessions; ++i)
    if (n_host[i] < 0 || n_host[i] >= ((int64_t)1 << 31)) return 0;
  return scan_topk_ws_bytes(n_host, n_sessions, hkv, hq, group);
}

static int32_t check_scan_topk_session(const fathom_session &s, const char *who) {
  REQUIRE(s.n >= 0 && s.n < ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "%s: n must be in [0, 2^31) (got %lld)", who, (long long)s.n);
  REQUIRE(s.idx && s.vals, FATHOM_ERR_INVALID_ARG, "%s: null output", who);
  if (int32_t rc = check_plane_words(s, who)) return rc;
  if (s.n == 0) return FATHOM_OK;
  REQUIRE(s.planes && s.lo && s.hi && s.q && s.plan, FATHOM_ERR_INVALID_ARG,
          "%s: null pointer", who);
  return FATHOM_OK;
}

static int32_t scan_topk_common(const fathom_session *sessions, int32_t n_sessions,
                                int32_t hkv, int32_t d, int32_t hq, int32_t group, int32_t k,
                                void *ws, int64_t ws_bytes, void *stream, const char *who,
                                int64_t rs = 0, int32_t meta_bits = 8) {
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  if (int32_t rc = check_topk_common(hq, group, k, who)) return rc;
  ScanSession ss[FATHOM_MAX_SESSIONS];
  int32_t *idx[FATHOM_MAX_SESSIONS];
  float *vals[FATHOM_MAX_SESSIONS];
  int64_t ns[FATHOM_MAX_SESSIONS];
  for (int32_t i = 0; i < n_sessions; ++i) {
    if (int32_t rc = check_scan_topk_session(sessions[i], who)) return rc;
    fathom_session c = sessions[i];
    c.logits = nullptr;
    c.ld_logits = 0;
    ss[i] = to_scan(c);
    ss[i].sample = nullptr;
    ss[i].thr = nullptr;
    ss[i].cand = nullptr;
    ss[i].seg_cnt = nullptr;
    ss[i].redo = nullptr;
    ss[i].rs = rs;
    ss[i].meta_bits = meta_bits;
    idx[i] = sessions[i].idx;
    vals[i] = sessions[i].vals;
    ns[i] = sessions[i].n;
  }
  const int64_t need = scan_topk_ws_bytes(ns, n_sessions, hkv, hq, group);
  REQUIRE(ws && ws_bytes >= need, FATHOM_ERR_WORKSPACE,
          "%s: workspace of %lld bytes needed (got %lld)", who, (long long)need,
          (long long)ws_bytes);
  return launch_scan_topk(ss, idx, vals, n_sessions, hkv, hq, group, k, ws, as_stream(stream));
}

int32_t fathom_scan_topk(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
                         int32_t hkv, int32_t d, const float *q, const uint8_t *plan,
                         int32_t hq, const uint8_t *meta, float meta_scale, int32_t group,
                         int32_t k, int32_t *idx, float *vals, void *ws, int64_t ws_bytes,
                         void *stream) {
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.meta = meta;
  s.meta_scale = meta_scale;
  s.idx = idx;
  s.vals = vals;
  return scan_topk_common(&s, 1, hkv, d, hq, group, k, ws, ws_bytes, stream,
                          "fathom_scan_topk");
}

int32_t fathom_scan_topk_meta4(const uint32_t *planes, const float *lo, const float *hi,
                               int64_t n, int32_t hkv, int32_t d, const float *q,
                               const uint8_t *plan, int32_t hq, const uint8_t *meta4,
                               float meta_scale, int32_t group, int32_t k, int32_t *idx,
                               float *vals, void *ws, int64_t ws_bytes, void *stream) {
  REQUIRE(meta4 || n == 0, FATHOM_ERR_INVALID_ARG, "fathom_scan_topk_meta4: null side stream");
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.meta = meta4;
  s.meta_scale = meta_scale;
  s.idx = idx;
  s.vals = vals;
  return scan_topk_common(&s, 1, hkv, d, hq, group, k, ws, ws_bytes, stream,
                          "fathom_scan_topk_meta4", 0, 4);
}

int32_t fathom_scan_topk_blocked(const uint32_t *planes, const float *lo, const float *hi,
                                 int64_t range_stride, int64_t n, int32_t hkv, int32_t d,
                                 const float *q, const uint8_t *plan, int32_t hq,
                                 int64_t plane_words_, int32_t group, int32_t k, int32_t *idx,
                                 float *vals, void *ws, int64_t ws_bytes, void *stream) {
  if (int32_t rc = check_range_stride(range_stride, n, "fathom_scan_topk_blocked")) return rc;
  fathom_session s{};
  s.planes = planes;
  s.lo = lo;
  s.hi = hi;
  s.n = n;
  s.q = q;
  s.plan = plan;
  s.idx = idx;
  s.vals = vals;
  s.plane_words = plane_words_;
  return scan_topk_common(&s, 1, hkv, d, hq, group, k, ws, ws_bytes, stream,
                          "fathom_scan_topk_blocked", range_stride);
}

int32_t fathom_scan_topk_batched(const fathom_session *sessions, int32_t n_sessions,
                                 int32_t hkv, int32_t d, int32_t hq, int32_t group, int32_t k,
                                 void *ws, int64_t ws_bytes, void *stream) {
  REQUIRE(sessions, FATHOM_ERR_INVALID_ARG, "fathom_scan_topk_batched: null sessions");
  REQUIRE(n_sessions >= 1 && n_sessions <= FATHOM_MAX_SESSIONS, FATHOM_ERR_INVALID_ARG,
          "fathom_scan_topk_batched: n_sessions must be in [1, %d]", FATHOM_MAX_SESSIONS);
  return scan_topk_common(sessions, n_sessions, hkv, d, hq, group, k, ws, ws_bytes, stream,
                          "fathom_scan_topk_batched");
}

int32_t fathom_read_prefixes(const uint32_t *planes, int64_t n, int32_t hkv, int32_t d,
                             const uint8_t *plan, int32_t hq, uint8_t *out, void *stream) {
  REQUIRE(planes && plan && out, FATHOM_ERR_INVALID_ARG, "fathom_read_prefixes: null pointer");
  REQUIRE(n >= 0 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_read_prefixes: bad n");
  if (int32_t rc = check_heads(hq, hkv)) return rc;
  if (int32_t rc = check_d(d)) return rc;
  return launch_read_prefixes(planes, n, hkv, plan, hq, out, as_stream(stream));
}

int32_t fathom_plan_stats(const uint8_t *plan_host, int32_t hq, int32_t d, int32_t group,
                          uint32_t *hist, uint32_t *union_bits) {
  REQUIRE(plan_host && hist, FATHOM_ERR_INVALID_ARG, "fathom_plan_stats: null pointer");
  REQUIRE(hq >= 1 && d >= 1 && group >= 1 && hq % group == 0, FATHOM_ERR_INVALID_ARG,
          "fathom_plan_stats: bad shape");
  for (int t = 0; t < 5; ++t) hist[t] = 0;
  for (int32_t h = 0; h < hq; ++h)
    for (int32_t c = 0; c < d; ++c) {
      const uint8_t t = plan_host[(int64_t)h * d + c];
      REQUIRE(t <= 4, FATHOM_ERR_INVALID_ARG, "fathom_plan_stats: depth %d > 4", (int)t);
      ++hist[t];
    }
  if (union_bits) {
    for (int32_t g = 0; g < hq / group; ++g) {
      uint32_t bits = 0;
      for (int32_t c = 0; c < d; ++c) {
        uint8_t u = 0;
        for (int32_t j = 0; j < group; ++j) {
          const uint8_t t = plan_host[(int64_t)(g * group + j) * d + c];
          u = t > u ? t : u;
        }
        bits += u;
      }
      union_bits[g] = bits;
    }
  }
  return FATHOM_OK;
}

int32_t fathom_probe_read(const void *src, int64_t bytes, uint32_t *out, int32_t blocks,
                          void *stream) {
  REQUIRE(src && out, FATHOM_ERR_INVALID_ARG, "fathom_probe_read: null pointer");
  REQUIRE(bytes > 0 && bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0,
          FATHOM_ERR_INVALID_ARG, "fathom_probe_read: need 16-byte aligned, 16-byte sized");
  REQUIRE(blocks >= 0, FATHOM_ERR_INVALID_ARG, "fathom_probe_read: blocks < 0");
  return launch_probe_read(src, bytes, out, blocks, as_stream(stream));
}

int32_t fathom_probe_scan_traffic(const uint32_t *planes, int64_t n, int32_t hkv,
                                  const uint8_t *depth, int32_t rows_out, float *out,
                                  int64_t ld, uint32_t *sink, void *stream) {
  REQUIRE(planes && depth && sink, FATHOM_ERR_INVALID_ARG,
          "fathom_probe_scan_traffic: null pointer");
  REQUIRE(n > 0 && n % 2048 == 0 && n <= ((int64_t)1 << 31), FATHOM_ERR_INVALID_ARG,
          "fathom_probe_scan_traffic: n must be a positive multiple of 2048");
  REQUIRE(hkv >= 1 && hkv <= 64, FATHOM_ERR_INVALID_ARG, "fathom_probe_scan_traffic: hkv");
  REQUIRE(rows_out >= 0 && rows_out <= 16, FATHOM_ERR_INVALID_ARG,
          "fathom_probe_scan_traffic: rows_out must be 0..16");
  REQUIRE(rows_out == 0 || (out && ld >= n), FATHOM_ERR_INVALID_ARG,
          "fathom_probe_scan_traffic: out must hold hkv*rows_out rows of ld >= n");
  REQUIRE((reinterpret_cast<uintptr_t>(planes) & 15) == 0 &&
              (rows_out == 0 || ((reinterpret_cast<uintptr_t>(out) & 15) == 0 && ld % 4 == 0)),
          FATHOM_ERR_INVALID_ARG, "fathom_probe_scan_traffic: planes and out rows need 16-byte alignment");
  return launch_probe_scan_traffic(planes, n, hkv, depth, rows_out, out, ld, sink,
                                   as_stream(stream));
}

}  // extern "C"
