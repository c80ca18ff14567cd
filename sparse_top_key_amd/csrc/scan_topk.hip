// Scan and top-k in one call (explainer, problem statement: each decode step
// scores all n keys and keeps the top k).  The result is the one of
// fathom_scan followed by fathom_topk; the logits of all keys are only
// written when a row needs them.
//
// With device-resident planes the steps are:
//   1. sample scan    logits of 8 tiles (16384 keys) spread over each row,
//   2. threshold      per output row, a key T expected to leave ~2.5k of the
//                     row's n scores at or above it (all keys when n <= 8192),
//   3. candidate scan every key scored again, the (score key, index) words of
//                     those >= T stored in the row's candidate segment of the
//                     scan block (block-local counters in LDS, no global
//                     atomics),
//   4. final          the exact top k of each row whose candidate count lies
//                     in [k, 8192], ranked and written; other rows flagged,
//   5. redo scan      full logits of the flagged rows' kv heads, one block
//                     per kv head (blocks of unflagged kv heads return at
//                     once),
//   6. redo final     exact top k of the flagged rows from those logits.
// Every score >= T is a candidate, so a row with k..8192 candidates holds
// its exact top k; the redo steps cover every other row.  Steps 5-6 cost one
// early-exiting launch each when no row is flagged.
//
// Planes in pinned host memory, sessions above 2^25 keys, or groups other
// than 1 and hq/hkv <= 4: the logits go to the workspace and fathom_topk's
// kernels run on them.
#include <algorithm>

#include "fathom_internal.h"

namespace fathom {
namespace {

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }
int64_t ld_pad(int64_t n) { return std::max<int64_t>(64, (n + 63) / 64 * 64); }

// Valid keys among the sampled tiles of a row of n keys (only the last
// sampled tile can be partial).
int64_t sampled_keys(int64_t n) {
  const int64_t nt = (n + kBlockKeys - 1) / kBlockKeys;
  const int64_t ns = std::min<int64_t>(nt, kSampleTiles);
  int64_t m = 0;
  for (int64_t j = 0; j < ns; ++j) {
    const int64_t t = j * nt / ns;
    m += std::min<int64_t>(kBlockKeys, n - t * kBlockKeys);
  }
  return m;
}

struct Layout {
  int64_t topk_off, seg_off, fcand_off, sample_off, table_off, table_bytes, logits_off, total;
  int64_t out_rows, redo_slots;
};

Layout layout(const int64_t *n, int32_t n_sess, int32_t hkv, int32_t hq, int32_t group) {
  Layout L;
  L.out_rows = (int64_t)n_sess * (hq / group);
  L.redo_slots = std::max<int64_t>(L.out_rows, (int64_t)n_sess * hkv);
  L.topk_off = 0;
  L.seg_off = align256(topk_ws_bytes(L.out_rows, L.redo_slots));
  L.fcand_off = L.seg_off + align256(L.out_rows * kMaxSeg * (int64_t)sizeof(uint32_t));
  L.sample_off = L.fcand_off + align256(L.out_rows * kFusedCap * (int64_t)sizeof(uint64_t));
  L.table_off =
      L.sample_off + align256((int64_t)n_sess * hq * kSampleKeys * (int64_t)sizeof(float));
  L.table_bytes = align256(scan_table_bytes(hkv, hq));
  L.logits_off = L.table_off + (int64_t)n_sess * L.table_bytes;
  int64_t logits = 0;
  for (int32_t s = 0; s < n_sess; ++s)
    logits += align256((int64_t)hq * ld_pad(n[s]) * (int64_t)sizeof(float));
  L.total = L.logits_off + logits;
  return L;
}

}  // namespace

int64_t scan_topk_ws_bytes(const int64_t *n, int32_t n_sess, int32_t hkv, int32_t hq,
                           int32_t group) {
  return layout(n, n_sess, hkv, hq, group).total;
}

int32_t launch_scan_topk(const ScanSession *in, int32_t *const *idx, float *const *vals,
                         int32_t n_sess, int32_t hkv, int32_t hq, int32_t group, int32_t k,
                         void *ws, hipStream_t s) {
  int64_t ns[FATHOM_MAX_SESSIONS];
  for (int32_t j = 0; j < n_sess; ++j) ns[j] = in[j].n;
  const Layout L = layout(ns, n_sess, hkv, hq, group);
  char *w = static_cast<char *>(ws);
  TopkWs tw = topk_ws_carve(w + L.topk_off, L.out_rows, L.redo_slots);
  tw.seg_cnt = reinterpret_cast<uint32_t *>(w + L.seg_off);
  tw.fcand = reinterpret_cast<uint64_t *>(w + L.fcand_off);
  const int32_t rows_per_sess = hq / group;
  const int32_t rows_per_kv = std::max(1, rows_per_sess / hkv);

  // per-session views of the workspace; sessions without keys skip the scans
  ScanSession sc[FATHOM_MAX_SESSIONS];
  TopkSession fin[FATHOM_MAX_SESSIONS], thr[FATHOM_MAX_SESSIONS];
  int32_t m = 0;
  int64_t logits_off = L.logits_off;
  for (int32_t j = 0; j < n_sess; ++j) {
    ScanSession c = in[j];
    c.ld = ld_pad(in[j].n);
    c.logits = reinterpret_cast<float *>(w + logits_off);
    logits_off += align256((int64_t)hq * c.ld * (int64_t)sizeof(float));
    c.sample = reinterpret_cast<float *>(w + L.sample_off) + (int64_t)j * hq * kSampleKeys;
    const int64_t row0 = (int64_t)j * rows_per_sess;
    c.thr = tw.thr + row0;
    c.cand = tw.fcand + row0 * kFusedCap;
    c.seg_cnt = tw.seg_cnt + row0 * kMaxSeg;
    c.redo = nullptr;
    c.table = reinterpret_cast<uint8_t *>(w + L.table_off + (int64_t)j * L.table_bytes);
    c.table_mode = kTableRead;
    fin[j] = TopkSession{c.logits, in[j].n, c.ld, idx[j], vals[j], in[j].n, 0};
    thr[j] = TopkSession{c.sample, sampled_keys(in[j].n), kSampleKeys, idx[j], vals[j],
                         in[j].n, 0};
    if (in[j].n > 0) {
      sc[m] = c;
      sc[m].redo = tw.redo + (int64_t)j * hkv;  // used by the redo scan only
      ++m;
    }
  }
  // plain: no recompute flags; the sample scan stores the slot tables, the
  // candidate and recompute scans load them
  ScanSession plain[FATHOM_MAX_SESSIONS], first[FATHOM_MAX_SESSIONS];
  for (int32_t j = 0; j < m; ++j) {
    plain[j] = sc[j];
    plain[j].redo = nullptr;
    first[j] = plain[j];
    first[j].table_mode = kTableWrite;
  }

  // one residency query per session for the whole call
  if (!resolve_residency(sc, m)) return FATHOM_ERR_INVALID_ARG;
  for (int32_t j = 0; j < m; ++j) plain[j].residency = first[j].residency = sc[j].residency;
  const bool group_ok = group == 1 || (group == hq / hkv && group <= 4);
  if (!group_ok || (m > 0 && !scan_can_fuse(sc, m))) {
    for (int32_t j = 0; j < m; ++j) plain[j].table_mode = kTableNone;
    if (m > 0)
      if (int32_t rc = launch_scan(plain, m, hkv, hq, s)) return rc;
    return launch_topk(fin, n_sess, rows_per_sess, group, k, tw, s, kTopkAll);
  }
  if (m > 0)
    if (int32_t rc = launch_scan(first, m, hkv, hq, s, kScanSample)) return rc;
  if (int32_t rc = launch_topk(thr, n_sess, rows_per_sess, group, k, tw, s, kTopkThreshold,
                               rows_per_kv, hkv))
    return rc;
  int32_t nseg[FATHOM_MAX_SESSIONS];
  if (m > 0)
    if (int32_t rc = launch_scan(plain, m, hkv, hq, s, group == 1 ? kScanCand : kScanCandGroup,
                                 nseg))
      return rc;
  for (int32_t j = 0, i = 0; j < n_sess; ++j) fin[j].nseg = in[j].n > 0 ? nseg[i++] : 0;
  if (int32_t rc = launch_topk(fin, n_sess, rows_per_sess, group, k, tw, s, kTopkFusedFinal,
                               rows_per_kv, hkv))
    return rc;
  if (m > 0)
    if (int32_t rc = launch_scan(sc, m, hkv, hq, s, kScanLogits, nullptr, true)) return rc;
  return launch_topk(fin, n_sess, rows_per_sess, group, k, tw, s, kTopkRedoFinal, rows_per_kv,
                     hkv);
}

}  // namespace fathom
