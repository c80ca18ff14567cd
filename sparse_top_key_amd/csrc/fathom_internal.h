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
constexpr int kSampleTiles = 32;        // 2048-key tiles a fused call scores first
// The threshold's subsample of a sampled tile: the first 64 of every 256 keys
// (512 per tile, 16384 per row at 32 tiles), each as the top 16 bits of its
// order-preserving score key (0 marks a key past the end of the row).
constexpr int kSampleSub = 512;
constexpr int kSubKeys = kSampleTiles * kSampleSub;
// Sampled tile j of ns among nt (ns <= nt): the middle tile of the j-th of ns
// equal strata of the row (all tiles when ns == nt).  Centres, not starts: in
// a row whose score scale drifts along the sequence, a stratum's first tile
// is its least (or most) extreme one, which biases the threshold estimate.
__host__ __device__ inline int64_t sample_tile(int64_t j, int64_t ns, int64_t nt) {
  return (2 * j + 1) * nt / (2 * ns);
}
constexpr int kCntStride = 32;          // candidate counters, one 128-byte line each
constexpr int kMaxGH = 4;               // query heads per scan launch chunk
// Candidate store of the fused call: per output row, one segment per scan
// block of the row's kv head (at most kMaxSeg), kFusedCap words in all; a
// block whose candidates outgrow its segment puts the rest in the row's
// overflow list (kCandCap words, one global counter per row).
constexpr int kMaxSeg = 1024;
constexpr int kFusedCap = 32768;

// Compute units of the current device (queried once per device).
int device_cus();

// Thread-local error text behind fathom_last_error().
void set_error(const char *fmt, ...);
int32_t hip_fail(hipError_t e, const char *what);

inline int64_t plane_words(int64_t n) { return 64 * ((n + kBlockKeys - 1) / kBlockKeys); }

// Scores as order-preserving unsigned keys (after adding +0, so -0 ranks as
// +0), and the 64-bit candidate words (key, ~index): larger word = higher
// score, then lower index.
__device__ __forceinline__ uint32_t to_key(float x) {
  const uint32_t u = __float_as_uint(__fadd_rn(x, 0.0f));
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t compose(uint32_t key, int64_t i) {
  return ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)i);
}

// Top-k bookkeeping carved from a caller's workspace: per output row a
// threshold key, a candidate counter (own cache line), a redo flag and
// kCandCap candidate words; per (session, kv head) a recompute flag.
struct TopkWs {
  uint32_t *thr, *cnt, *flag, *redo;
  uint64_t *cand;
  uint32_t *seg_cnt;    // fused final only: [rows][kMaxSeg]
  uint64_t *fcand;      // fused final only: [rows][kFusedCap]
  uint32_t *redo_done;  // fused threshold only: [session][hkv][redo_chunks], zeroed there
  int32_t redo_chunks;  // head chunks per kv head
};
int64_t topk_ws_bytes(int64_t out_rows, int64_t redo_slots);
TopkWs topk_ws_carve(void *ws, int64_t out_rows, int64_t redo_slots);

// ---- pack -------------------------------------------------------------------
// rs: 0 for one range per channel (lo, hi [hkv][d]); > 0 for one range per
// 2048-key block (lo, hi [hkv][rs][d], rs >= the number of blocks).
int64_t pack_workspace_bytes(int64_t n, int32_t hkv);
int64_t pack_blocked_workspace_bytes(int64_t n, int32_t hkv);
int32_t launch_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                    int64_t stride_tok, int64_t stride_head, uint32_t *planes,
                    float *lo, float *hi, int64_t rs, float *sigma2, void *ws,
                    hipStream_t s);

// ---- plan -------------------------------------------------------------------
int32_t launch_plan(const float *q, int32_t hq, int32_t hkv,
                    const float *sigma2, const int32_t *budget_host,
                    uint8_t *plan, hipStream_t s);
int32_t launch_plan_rd(const float *q, int32_t hq, int32_t hkv,
                       const float *sigma2, const int32_t *budget_host,
                       uint8_t *plan, hipStream_t s);
int32_t launch_plan_group(const float *q, int32_t hq, int32_t hkv,
                          const float *sigma2, const int32_t *budget_host,
                          uint8_t *plan, hipStream_t s);
int32_t launch_plan_fixed(const float *q, int32_t hq, int32_t r, uint8_t *plan,
                          hipStream_t s);

// ---- calibrated allocation -----------------------------------------------------
int32_t launch_code_hist(const uint32_t *planes, int64_t n, int32_t hkv, int64_t W,
                         uint32_t *hist, hipStream_t s);
int32_t launch_plan_calibrated(const float *q, int32_t hq, int32_t hkv, const float *lo,
                               const float *hi, const uint32_t *hist,
                               const int32_t *budget_host, uint8_t *plan, bool per_group,
                               hipStream_t s);

// ---- append -------------------------------------------------------------------
// rs > 0: per-block ranges; the blocks the call starts get theirs first.
int32_t launch_append(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                      int64_t stride_tok, int64_t stride_head, int64_t n_old,
                      uint32_t *planes, int64_t W, float *lo, float *hi, int64_t rs,
                      uint32_t *clamped, hipStream_t s);

// ---- sparse attention -------------------------------------------------------
int64_t attn_workspace_bytes(int32_t hq, int32_t k);
int32_t launch_attention(const float *q, int32_t hq, int32_t hkv, const void *kc,
                         const void *vc, int32_t dtype, int64_t n, int64_t stride_tok,
                         int64_t stride_head, const int32_t *idx, int32_t group, int32_t k,
                         float scale, float *out, float *lse, void *ws, hipStream_t s);

// ---- scan -------------------------------------------------------------------
struct ScanSession {
  const uint32_t *planes;
  const float *lo, *hi;
  int64_t n;
  const float *q;
  const uint8_t *plan;
  const uint8_t *meta;
  float meta_scale;
  int32_t meta_bits;      // side stream: 8 (uint8 [hkv][n]), 4 (nibbles [hkv][ceil(n/2)]); 0 = 8
  float *logits;
  int64_t ld;
  // fused scan + top-k (unused by plain scans)
  uint16_t *sample;       // [rows][kSubKeys] the sampled tiles' subsample (16-bit keys)
  const uint32_t *thr;    // [rows] threshold keys of the session's output rows
  uint64_t *cand;         // [rows][kFusedCap] candidate segments
  uint32_t *seg_cnt;      // [rows][kMaxSeg] candidates found by each block
  uint32_t *ovf_cnt;      // [rows] (stride kCntStride): candidates past their segment
  uint64_t *ovf;          // [rows][kCandCap] ... stored here, in arrival order
  // recompute scan of a fused call (redo_done set): only (kv head, head
  // chunk)s with a row whose candidate count (over its nseg segments) lies
  // outside [out_k, kCandCap] are scanned, and the last block of each ranks
  // those rows into the outputs
  uint32_t *redo_done;    // [hkv][head chunks] blocks finished (zeroed earlier in the call)
  int32_t nseg;           // candidate segments per row (the candidate scan's blocks per kv head)
  // set by the fused final's blocks (launch_scan's final_rows) for such rows
  uint32_t *redo;         // [hkv] kv heads with a recomputed row
  uint32_t *row_flag;     // [rows] recomputed rows
  int32_t *out_idx;       // [rows][out_k]
  float *out_vals;        // [rows][out_k]
  int32_t out_k;
  int32_t out_group;      // 1: a row per query head; hq / hkv: a row per kv head
  uint8_t *table;         // slot tables of the session's kv heads, or null
  int32_t table_mode;     // ScanTable: what the scan does with them
  int32_t residency;      // planes: 0 unknown (queried), 1 device, 2 pinned host
  int64_t W;              // plane row length in words; 0: plane_words(n)
  int64_t rs;             // 0: lo, hi [hkv][d]; > 0: per 2048-key block, [hkv][rs][d]
};
inline int64_t sess_words(const ScanSession &s) { return s.W > 0 ? s.W : plane_words(s.n); }
// Slot tables (matrix-core scan): built in each block (kTableNone), built and
// also stored for later scans of the same call (kTableWrite), or loaded from
// what an earlier scan of the call stored (kTableRead).
enum ScanTable { kTableNone = 0, kTableWrite = 1, kTableRead = 2 };
// Bytes of the slot tables of one session (all its kv heads and head chunks).
int64_t scan_table_bytes(int32_t hkv, int32_t hq);
// What a scan writes: every logit (into logits; in a fused call's recompute
// scan, only those of kv heads with a row to recompute), the logits of the sampled tiles (into sample), or the
// (score key, index) words of the keys whose score key reaches the row's
// threshold (into cand): kScanCand with one output row per query head,
// kScanCandGroup with one row per kv head scored by the sum of its
// hq / hkv (<= 4) query heads.
enum ScanMode { kScanLogits = 0, kScanSample = 1, kScanCand = 2, kScanCandGroup = 3 };
// nseg_out (candidate mode, optional): per session, the blocks per kv head,
// i.e. the candidate segments of each row.  one_block_per_head: a single
// block per (session, kv head) takes all its tiles (a grid of hkv blocks per
// session, for recomputations that are usually skipped).  final_rows
// (recompute scan of a fused call): the launch also runs the fused final of
// the sessions' final_rows output rows each, one block per row ahead of the
// scan blocks (the sessions' cand, seg_cnt, ovf, out_* and flags).
int32_t launch_scan(const ScanSession *sess, int32_t n_sess, int32_t hkv,
                    int32_t hq, hipStream_t s, int32_t mode = kScanLogits,
                    int32_t *nseg_out = nullptr, bool one_block_per_head = false,
                    int32_t final_rows = 0);
// Whether launch_scan can run the sample and candidate modes on these
// sessions (planes in device memory, at most 2^25 keys each).
bool scan_can_fuse(const ScanSession *sess, int32_t n_sess);
// Queries the residency of every session's planes once and records it in the
// sessions (later launch_scan calls on them skip the query); false (error
// set) if some are neither device nor pinned host memory.
bool resolve_residency(ScanSession *sess, int32_t n_sess);
int32_t launch_read_prefixes(const uint32_t *planes, int64_t n, int32_t hkv,
                             const uint8_t *plan, int32_t hq, uint8_t *out,
                             hipStream_t s);

// ---- top-k ------------------------------------------------------------------
struct TopkSession {
  const float *scores;  // first input row of the session
  const uint16_t *sub;  // threshold stage: first subsample row (kSubKeys apart), else null
  int64_t n, ld;
  int32_t *idx;
  float *vals;
  int64_t n_full;       // keys of the row the scores were sampled from (n if not sampled)
  int32_t nseg;         // fused final: candidate segments per row (kFusedCap / nseg each)
};
int64_t topk_workspace_bytes(int32_t out_rows);
// Plain: sample -> compact -> final over the scores.  Fused: threshold from
// scores holding only the sampled logits, then (after the candidate scan) a
// final pass that flags rows whose candidate count is out of range (the
// recompute scan ranks those).
enum TopkStage { kTopkAll = 0, kTopkThreshold = 1, kTopkFusedFinal = 2 };
int32_t launch_topk(const TopkSession *sess, int32_t n_sess, int32_t rows_per_sess,
                    int32_t group, int32_t k, const TopkWs &w, hipStream_t s,
                    int32_t stage = kTopkAll, int32_t rows_per_kv = 1, int32_t hkv = 1);

// ---- no-allocation scratch (noalloc.hip) ------------------------------------
// Device address of the current device's static scratch array (looked up once
// per device) and its size in bytes.
int32_t noalloc_scratch(void **ptr);
int64_t noalloc_scratch_bytes();

// ---- scan + top-k -----------------------------------------------------------
int64_t scan_topk_ws_bytes(const int64_t *n, int32_t n_sess, int32_t hkv, int32_t hq,
                           int32_t group);
int32_t launch_scan_topk(const ScanSession *in, int32_t *const *idx, float *const *vals,
                         int32_t n_sess, int32_t hkv, int32_t hq, int32_t group, int32_t k,
                         void *ws, hipStream_t s);

// ---- probe ------------------------------------------------------------------
int32_t launch_probe_scan_traffic(const uint32_t *planes, int64_t n, int32_t hkv,
                                  const uint8_t *depth, int32_t rows_out, float *out,
                                  int64_t ld, uint32_t *sink, hipStream_t s);
int32_t launch_probe_read(const void *src, int64_t bytes, uint32_t *out,
                          int32_t blocks, hipStream_t s);

}  // namespace fathom
