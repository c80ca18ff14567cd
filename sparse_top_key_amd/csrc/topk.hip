// Top-k key selection per decode step (explainer, problem statement: each
// generated token keeps the top k of the n scored keys).  Ranking: score
// descending, then index ascending; results are those of a full sort.
//
// Three launches per call (MI355X-first design; the pages give none):
//   topk_sample   one block per output row: reads a sample of the row
//                 (64-score runs spread evenly, about 16K scores; or, in the
//                 fused call, the row's subsample of 16-bit score keys) and
//                 picks a threshold key T expected to leave about 2.5k
//                 scores at or above it, by two 11-bit radix digits below
//                 the bits all sampled keys share (fused call: one histogram
//                 of the three binades below the largest key when that
//                 suffices).  Rows of at most 8192 scores take T = 0 (all).
//   topk_compact  the whole grid streams every row once and appends the
//                 (score key, index) words >= T to the row's candidate list
//                 (staged in LDS, one global atomic per block).
//   topk_final    one block per output row: if the candidates hold at least k
//                 and at most 8192 words they contain the exact top k (every
//                 score >= T is present).  The winners are ranked without a
//                 sort: words are bucketed on the 12 bits below their common
//                 prefix and each takes its bucket's offset plus the number of
//                 larger words in its bucket (a radix select plus a merge sort
//                 of in-wave bitonic runs when a bucket is too large).  Other
//                 rows are recomputed exactly: a 3-pass radix select over the
//                 whole row finds the k-th key, an index-ordered pass gathers
//                 the winners (ties at the k-th key by lowest index), and the
//                 same ranking orders them (select.h holds these steps).
// The fused scan + top-k call reuses these kernels in stages: the threshold
// from the sampled subsample, and a final over the candidate segments the
// scan wrote (rows out of range are flagged instead of recomputed; the
// recompute scan ranks them once their logits exist).
// Scores map to order-preserving uint32 keys after adding +0 (so -0 ranks as
// +0); a GQA group's score is its rows' fp32 scores added in fp64, in row
// order, rounded once.
#include "fathom_internal.h"
#include "select.h"

namespace fathom {
namespace {

constexpr int kBig = kSelThreads;     // threads of the per-row kernels
constexpr int kCompactThreads = 256;
constexpr int kCompactChunk = 16384;  // scores per compact block
constexpr int kRun = 64;              // contiguous scores per sample run
constexpr int kStage = 2048;           // candidates staged per compact block

struct TopkSess {
  const float *scores;
  const uint16_t *sub;  // threshold stage: subsample rows (kSubKeys apart)
  int64_t n, ld;
  int32_t *idx;
  float *vals;
  int64_t n_full;
  int32_t nseg;
};

struct TopkArgs {
  TopkSess s[kSessPerLaunch];
  int32_t rows_per_sess, group, k;
  int32_t stage;        // TopkStage
  int32_t rows_per_kv;  // output rows per kv head (redo flags)
  int32_t hkv;
  uint32_t *thr;
  uint32_t *cnt;        // stride kCntStride
  uint32_t *flag;
  uint32_t *redo;       // [session][hkv] of this launch
  uint64_t *cand;
  uint32_t *seg_cnt;    // fused final: [rows][kMaxSeg]
  uint64_t *fcand;      // fused final: [rows][kFusedCap]
  uint32_t *redo_done;  // fused threshold: [session][hkv][redo_chunks] (zeroed)
  int32_t redo_chunks;
};

struct RowRef {
  const TopkSess *s;
  const float *row;
};

__device__ __forceinline__ RowRef row_ref(const TopkArgs &a, int o) {
  const int si = o / a.rows_per_sess;
  const int r = o % a.rows_per_sess;
  RowRef ref;
  ref.s = &a.s[si];
  ref.row = a.s[si].scores + (int64_t)r * a.group * a.s[si].ld;
  return ref;
}


// ---- sample -> threshold -----------------------------------------------------
// Max, min and sum over the block (16 waves).
__device__ void block_minmax_count(uint32_t &mx, uint32_t &mn, int &cnt, uint32_t *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
    cnt += __shfl_xor(cnt, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave] = mx;
    red[16 + wave] = mn;
    red[32 + wave] = (uint32_t)cnt;
  }
  __syncthreads();
  mx = 0;
  mn = 0xFFFFFFFFu;
  cnt = 0;
#pragma unroll
  for (int w = 0; w < kBig / 64; ++w) {
    mx = max(mx, red[w]);
    mn = min(mn, red[16 + w]);
    cnt += (int)red[32 + w];
  }
  __syncthreads();
}

// One block per output row: from a sample of the row (runs of 64 scores
// spread evenly, about 16K in all; or, in the fused threshold stage, the
// row's subsample of 16-bit keys), a threshold key T expected to leave about
// 2.5k of the row's n_full scores at or above it: the sample's keys are
// histogrammed on the 11 bits below their common prefix and T is the lower
// edge of the bin holding the rs-th largest.  Rows of at most 8192 scores
// take T = 0 (all).
__global__ __launch_bounds__(kBig) void topk_sample_kernel(TopkArgs a) {
  constexpr int kPer = (kSampleTarget + kRun + kBig - 1) / kBig;
  constexpr int kSubPer = kSubKeys / kBig;  // subsample keys per thread (fused stage)
  static_assert(kSubPer <= kPer && kSubPer == 16 && kSampleSub % kSubPer == 0, "subsample");
  __shared__ int hist[kHistBins];
  __shared__ int wave_tot[16];
  __shared__ int s_res[2];
  __shared__ uint32_t red[48];
  __shared__ int tile_cnt[kSampleTiles];   // fused threshold: per sampled tile
  __shared__ bool tile_out[kSampleTiles];
  const int o = blockIdx.x;
  const RowRef R = row_ref(a, o);
  const int64_t n = R.s->n, ld = R.s->ld, n_full = R.s->n_full;
  if (threadIdx.x == 0) {
    const int r = o % a.rows_per_sess, si = o / a.rows_per_sess;
    a.cnt[(int64_t)o * kCntStride] = 0;
    a.flag[o] = 0;
    a.redo[si * a.hkv + r / a.rows_per_kv] = 0;
    // the recompute scan's count of finished blocks of this row's (kv head,
    // head chunk)
    if (a.redo_done)
      a.redo_done[((int64_t)si * a.hkv + r / a.rows_per_kv) * a.redo_chunks +
                  (r % a.rows_per_kv) / kMaxGH] = 0;
  }
  if (n_full <= kCandCap) {
    if (threadIdx.x == 0) a.thr[o] = 0;
    return;
  }
  const bool tiled = a.stage == kTopkThreshold;
  int64_t stride = (n * kRun + kSampleTarget - 1) / kSampleTarget;
  stride = (stride + kRun - 1) / kRun * kRun;
  if (stride < kRun) stride = kRun;
  const int runs = (int)((n + stride - 1) / stride);
  const int m = runs * kRun;
  // every load of the thread in flight at once (one row: plain loads first,
  // keys after)
  uint32_t v[kPer];
  uint32_t okm = 0;
  if (tiled) {
    // 16 consecutive subsample keys per thread, all of one sampled tile (two
    // 16-byte loads); key 0 marks an entry past the end of the row, and the
    // key's low 16 bits are taken as 0 (T is then the lower edge of its
    // 16-bit bin)
    const uint16_t *sub = R.s->sub + (int64_t)(o % a.rows_per_sess) * kSubKeys;
    const int e0 = threadIdx.x * kSubPer;
    uint4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (e0 < n) {
      w0 = reinterpret_cast<const uint4 *>(sub + e0)[0];
      w1 = reinterpret_cast<const uint4 *>(sub + e0)[1];
    }
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t k16 = j < kSubPer ? (wd[j >> 1] >> (16 * (j & 1))) & 0xFFFFu : 0u;
      v[j] = k16 << 16;
      okm |= (uint32_t)(k16 != 0u) << j;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = threadIdx.x + j * kBig;
      const int64_t pos = (int64_t)(e / kRun) * stride + (e % kRun);
      okm |= (uint32_t)(e < m && pos < n) << j;
    }
  }
  if (!tiled && a.group == 1) {
    // unconditional loads (positions out of the sample read element 0, which
    // exists: n >= 1 here), so that all of them are issued before any wait
    float f[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = threadIdx.x + j * kBig;
      const int64_t pos = (int64_t)(e / kRun) * stride + (e % kRun);
      f[j] = R.row[((okm >> j) & 1) ? pos : 0];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = ((okm >> j) & 1) ? to_key(f[j]) : 0u;
  } else if (!tiled) {
    // group scores: rows added in fp64 in row order (as group_score does);
    // per row and half of the samples, every load is issued before the adds
    constexpr int kHalf = (kPer + 1) / 2;
#pragma unroll
    for (int j0 = 0; j0 < kPer; j0 += kHalf) {
      double acc[kHalf];
#pragma unroll
      for (int u = 0; u < kHalf; ++u) acc[u] = 0.0;
      for (int r = 0; r < a.group; ++r) {
        const float *rr = R.row + (int64_t)r * ld;
        float f[kHalf];
#pragma unroll
        for (int u = 0; u < kHalf; ++u) {
          const int j = j0 + u;
          const int e = threadIdx.x + j * kBig;
          const int64_t pos = (int64_t)(e / kRun) * stride + (e % kRun);
          f[u] = (j < kPer && ((okm >> j) & 1)) ? rr[pos] : rr[0];
        }
#pragma unroll
        for (int u = 0; u < kHalf; ++u) acc[u] = __dadd_rn(acc[u], (double)f[u]);
      }
#pragma unroll
      for (int u = 0; u < kHalf; ++u)
        if (j0 + u < kPer) v[j0 + u] = ((okm >> (j0 + u)) & 1) ? to_key((float)acc[u]) : 0u;
    }
  }
  // Fused threshold stage: the subsample row holds 512 keys of each sampled
  // tile, the middle tiles of equal stretches of the row.  A tile whose count
  // of sampled keys at or above T exceeds 4x its larger neighbour's (+8) holds a
  // local cluster of top keys (one stretch of the row, not a drift, which
  // changes smoothly from tile to tile): the sample then overstates the
  // cluster by the sampling ratio and T lands above almost all other keys.
  // Such tiles are left out and T is taken again from the others (the
  // cluster's own keys are still candidates: they lie above it).
  const int ntl = tiled ? (int)(n / kSampleSub) : 0;
  const int my_tile = threadIdx.x * kSubPer / kSampleSub;  // (tiled)
  uint32_t prefix = 0;
#pragma unroll 1
  for (int round = 0; round < 2; ++round) {
    uint32_t mx = 0, mn = 0xFFFFFFFFu;
    int cnt = __popc(okm);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if ((okm >> j) & 1) {
        mx = max(mx, v[j]);
        mn = min(mn, v[j]);
      }
    block_minmax_count(mx, mn, cnt, red);
    if (cnt == 0) {
      if (threadIdx.x == 0) a.thr[o] = 0;
      return;
    }
    // rank of the threshold inside the sample: ~2.5k of n_full at or above T
    int64_t rs = ((int64_t)5 * a.k * cnt + 2 * n_full - 1) / (2 * n_full);
    rs = rs < 1 ? 1 : (rs > cnt ? cnt : rs);
    int rem = (int)rs;
    // Fused stage with a positive largest score (in binade e >= 2): the keys
    // from the start of binade e - 2 up span three binades, which bins of
    // 2^14 key units split into 1536 (finer than the 16-bit keys); when at
    // least rs keys lie there, one histogram of them gives T = the rs-th
    // largest key (far fewer LDS atomics than a pass over every key).
    bool found = false;
    if (tiled && mx >= 0x80000000u + (2u << 23)) {
      const uint32_t lo = 0x80000000u | ((((mx >> 23) & 0xFFu) - 2u) << 23);
      constexpr int kWinShift = 14;
      for (int b = threadIdx.x; b < kHistBins; b += kBig) hist[b] = 0;
      if (threadIdx.x == 0) s_res[0] = -1;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (((okm >> j) & 1) && v[j] >= lo) atomicAdd(&hist[(v[j] - lo) >> kWinShift], 1);
      __syncthreads();
      int above = 0;
      const int d = find_digit(hist, kHistBins, rem, &above, wave_tot, s_res);
      if (d >= 0) {  // block-uniform
        prefix = lo + ((uint32_t)d << kWinShift);
        found = true;
      }
    }
    // Otherwise two 11-bit digits below the bits all sampled keys share: T =
    // the rs-th largest key with its bits below the second digit cleared.
    const uint32_t diff = mx ^ mn;
    const int hb = diff ? 31 - __clz(diff) : 0;  // highest bit in which keys differ
    int sh = hb > 10 ? hb - 10 : 0;
    if (!found) {
      prefix = sh + 11 >= 32 ? 0u : (mx >> (sh + 11)) << (sh + 11);
    }
    uint32_t pmask = sh + 11 >= 32 ? 0u : ~((1u << (sh + 11)) - 1u);
    for (int pass = 0; pass < 2 && !found; ++pass) {
      for (int b = threadIdx.x; b < kHistBins; b += kBig) hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (((okm >> j) & 1) && (v[j] & pmask) == prefix)
          atomicAdd(&hist[(v[j] >> sh) & (kHistBins - 1)], 1);
      __syncthreads();
      int above = 0;
      const int d = find_digit(hist, kHistBins, rem, &above, wave_tot, s_res);
      rem -= above;
      prefix |= (uint32_t)d << sh;
      pmask |= (uint32_t)(kHistBins - 1) << sh;
      if (sh == 0) break;
      // next digit: the 11 bits below (when fewer remain, it also spans bits
      // the matching keys share, which keeps its order)
      sh = sh > 11 ? sh - 11 : 0;
    }
    if (round == 1 || ntl < 3) break;
    // per-tile counts of sampled keys at or above T, then the outliers
    for (int t = threadIdx.x; t < ntl; t += kBig) tile_cnt[t] = 0;
    __syncthreads();
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += ((okm >> j) & 1) && v[j] >= prefix;
    if (mine) atomicAdd(&tile_cnt[my_tile], mine);
    __syncthreads();
    if (threadIdx.x == 0) s_res[0] = 0;
    __syncthreads();
    for (int t = threadIdx.x; t < ntl; t += kBig) {
      const int nb = max(t > 0 ? tile_cnt[t - 1] : 0, t + 1 < ntl ? tile_cnt[t + 1] : 0);
      const bool outlier = tile_cnt[t] > 4 * nb + 8;
      tile_out[t] = outlier;
      if (outlier) s_res[0] = 1;
    }
    __syncthreads();
    if (!s_res[0]) break;  // block-uniform
    if (tile_out[my_tile]) okm = 0;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.thr[o] = prefix;
}

// ---- stream the rows, keep scores >= T ----------------------------------------
// Candidates are staged in LDS and appended to the row's list with one global
// atomic per block (all rows' counters share a cache line, so per-wave global
// atomics would serialise in one L2 channel).  A block with more than kStage
// candidates sends the overflow straight to the global list.
__global__ __launch_bounds__(kCompactThreads) void topk_compact_kernel(TopkArgs a) {
  __shared__ uint64_t stage[kStage];
  __shared__ uint32_t s_n, s_base;
  const int o = blockIdx.y;
  const RowRef R = row_ref(a, o);
  const int64_t n = R.s->n, ld = R.s->ld;
  const int64_t base = (int64_t)blockIdx.x * kCompactChunk;
  if (base >= n) return;
  const uint32_t T = a.thr[o];
  uint32_t *cnt = a.cnt + (int64_t)o * kCntStride;
  uint64_t *cand = a.cand + (int64_t)o * kCandCap;
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool vec = a.group == 1 && ((reinterpret_cast<uintptr_t>(R.row) & 15) == 0);
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  constexpr int kIters = kCompactChunk / (kCompactThreads * 4);
  float4 pre[kIters];
  const bool full = vec && base + kCompactChunk <= n;
  if (full) {
    // every load of the chunk in flight at once
#pragma unroll
    for (int it = 0; it < kIters; ++it)
      pre[it] = *reinterpret_cast<const float4 *>(R.row + base + (int64_t)it * kCompactThreads * 4 +
                                                  threadIdx.x * 4);
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t i0 = base + (int64_t)it * kCompactThreads * 4 + threadIdx.x * 4;
    float v[4];
    if (full) {
      v[0] = pre[it].x; v[1] = pre[it].y; v[2] = pre[it].z; v[3] = pre[it].w;
    } else if (vec && i0 + 3 < n) {
      const float4 f = *reinterpret_cast<const float4 *>(R.row + i0);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = i0 + e < n ? group_score(R.row, ld, a.group, i0 + e) : 0.0f;
    }
    uint32_t key[4];
    bool pred[4];
    uint64_t bal[4];
    uint32_t total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[e] = to_key(v[e]);
      pred[e] = (i0 + e < n) && key[e] >= T;
      bal[e] = __ballot(pred[e]);
      total += __popcll(bal[e]);
    }
    if (total == 0) continue;
    uint32_t start = 0;
    if (lane == 0) start = atomicAdd(&s_n, total);
    start = __shfl(start, 0);
    // positions >= kStage of this batch go to the global list directly
    const uint32_t first_over = start > (uint32_t)kStage ? start : (uint32_t)kStage;
    const uint32_t over = start + total > first_over ? start + total - first_over : 0u;
    uint32_t gbase = 0;
    if (over) {
      if (lane == 0) gbase = atomicAdd(cnt, over);
      gbase = __shfl(gbase, 0);
    }
    uint32_t off = start;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (pred[e]) {
        const uint32_t pos = off + __popcll(bal[e] & below);
        const uint64_t c = compose(key[e], i0 + e);
        if (pos < (uint32_t)kStage) {
          stage[pos] = c;
        } else {
          const uint32_t g = gbase + (pos - first_over);
          if (g < (uint32_t)kCandCap) cand[g] = c;
        }
      }
      off += __popcll(bal[e]);
    }
  }
  __syncthreads();
  const uint32_t m = s_n < (uint32_t)kStage ? s_n : (uint32_t)kStage;
  if (m == 0) return;
  if (threadIdx.x == 0) s_base = atomicAdd(cnt, m);
  __syncthreads();
  const uint32_t b = s_base;
  for (uint32_t j = threadIdx.x; j < m; j += kCompactThreads)
    if (b + j < (uint32_t)kCandCap) cand[b + j] = stage[j];
}

// ---- exact selection of each row's top k -------------------------------------
__global__ __launch_bounds__(kBig) void topk_final_kernel(TopkArgs a) {
  __shared__ uint64_t s[kCandCap];
  __shared__ uint64_t win[kBuckCap];
  __shared__ int hist[kRankBins];
  __shared__ int above[kRankBins + 1];  // [kRankBins]: the big bucket (bucket_rank_out)
  __shared__ uint64_t red[kBig / 64];
  __shared__ int wave_tot[16];
  __shared__ int s_res[2];
  __shared__ int s_count;
  __shared__ int s_off[kMaxSeg + 1];
  const int o = blockIdx.x;
  const RowRef R = row_ref(a, o);
  const TopkSess &S = *R.s;
  const int r = o % a.rows_per_sess;
  const int64_t n = S.n, ld = S.ld;
  const int k = a.k;
  const int kk = (int)(n < k ? n : k);
  int32_t *idx = S.idx + (int64_t)r * k;
  float *vals = S.vals + (int64_t)r * k;
  if (a.stage == kTopkFusedFinal) {
    // too few or too many candidates: the row is flagged and recomputed from
    // full logits (by the last block of the recompute scan of its kv head)
    const FinalScratch X{s, win, hist, above, red, wave_tot, s_res, &s_count, s_off};
    if (!fused_final_row(a.fcand + (int64_t)o * kFusedCap, a.seg_cnt + (int64_t)o * kMaxSeg,
                         S.nseg, a.cand + (int64_t)o * kCandCap, a.cnt + (int64_t)o * kCntStride,
                         n, k, idx, vals, X) &&
        threadIdx.x == 0) {
      a.flag[o] = 1;
      a.redo[(o / a.rows_per_sess) * a.hkv + r / a.rows_per_kv] = 1;
    }
    return;
  }
  const uint32_t cnt = a.cnt[(int64_t)o * kCntStride];
  const bool fast = (n <= kCandCap) || (cnt >= (uint32_t)k && cnt <= (uint32_t)kCandCap);
  if (!fast) {
    // exact recomputation over the whole row
    const SelScratch X{win, s, hist, above, wave_tot, s_res, &s_count, red};
    exact_row_topk(R.row, ld, a.group, n, k, idx, vals, X);
    return;
  }
  if (threadIdx.x == 0) s_count = 0;
  const int m = (int)cnt;
  const uint64_t *cand = a.cand + (int64_t)o * kCandCap;
  for (int j = threadIdx.x; j < m; j += kBig) s[j] = cand[j];
  __syncthreads();
  if (kk > 0 && bucket_rank_out(s, m, kk, win, hist, above, wave_tot, s_res, red, idx, vals, k,
                                s + kBuckCap))
    return;
  if (kk > 0) {
    const uint64_t T = m > kk ? select_kth(s, m, kk, hist, wave_tot, s_res) : 0ull;
    for (int j = threadIdx.x; j < m; j += kBig)
      if (s[j] >= T) win[atomicAdd(&s_count, 1)] = s[j];
  }
  __syncthreads();
  // win[0..kk) holds the winners
  const uint64_t *sorted = sort_winners_desc(win, s, kk);
  write_out(idx, vals, k, sorted, kk);
}

}  // namespace

// Workspace: thr[rows] | flag[rows] | redo[redo_slots] | pad to 256 |
// cnt[rows][kCntStride] | cand[rows][kCandCap].
static int64_t small_bytes(int64_t out_rows, int64_t redo_slots) {
  return ((2 * out_rows + redo_slots) * (int64_t)sizeof(uint32_t) + 255) / 256 * 256;
}

int64_t topk_ws_bytes(int64_t out_rows, int64_t redo_slots) {
  return small_bytes(out_rows, redo_slots) + out_rows * kCntStride * (int64_t)sizeof(uint32_t) +
         out_rows * kCandCap * (int64_t)sizeof(uint64_t);
}

TopkWs topk_ws_carve(void *ws, int64_t out_rows, int64_t redo_slots) {
  char *w = static_cast<char *>(ws);
  TopkWs t;
  t.thr = reinterpret_cast<uint32_t *>(w);
  t.flag = t.thr + out_rows;
  t.redo = t.flag + out_rows;
  const int64_t small = small_bytes(out_rows, redo_slots);
  t.cnt = reinterpret_cast<uint32_t *>(w + small);
  t.cand = reinterpret_cast<uint64_t *>(w + small + out_rows * kCntStride * sizeof(uint32_t));
  t.seg_cnt = nullptr;
  t.fcand = nullptr;
  t.redo_done = nullptr;
  t.redo_chunks = 1;
  return t;
}

int64_t topk_workspace_bytes(int32_t out_rows) { return topk_ws_bytes(out_rows, out_rows); }

int32_t launch_topk(const TopkSession *sess, int32_t n_sess, int32_t rows_per_sess,
                    int32_t group, int32_t k, const TopkWs &w, hipStream_t s, int32_t stage,
                    int32_t rows_per_kv, int32_t hkv) {
  if (stage == kTopkAll) {  // redo flags unused: one slot per row
    hkv = rows_per_sess;
    rows_per_kv = 1;
  }
  for (int32_t s0 = 0; s0 < n_sess; s0 += kSessPerLaunch) {
    const int32_t cnt = std::min(kSessPerLaunch, n_sess - s0);
    const int32_t out_rows = cnt * rows_per_sess;
    TopkArgs a{};
    a.rows_per_sess = rows_per_sess;
    a.group = group;
    a.k = k;
    a.stage = stage;
    a.rows_per_kv = rows_per_kv;
    a.hkv = hkv;
    const int64_t rows_before = (int64_t)s0 * rows_per_sess;
    a.thr = w.thr + rows_before;
    a.flag = w.flag + rows_before;
    a.redo = w.redo + (int64_t)s0 * hkv;
    a.cnt = w.cnt + rows_before * kCntStride;
    a.cand = w.cand + rows_before * kCandCap;
    a.seg_cnt = w.seg_cnt ? w.seg_cnt + rows_before * kMaxSeg : nullptr;
    a.fcand = w.fcand ? w.fcand + rows_before * kFusedCap : nullptr;
    a.redo_done = stage == kTopkThreshold && w.redo_done
                      ? w.redo_done + (int64_t)s0 * hkv * w.redo_chunks
                      : nullptr;
    a.redo_chunks = w.redo_chunks;
    int64_t max_n = 0;
    for (int j = 0; j < cnt; ++j) {
      const TopkSession &in = sess[s0 + j];
      a.s[j].scores = in.scores;
      a.s[j].sub = in.sub;
      a.s[j].n = in.n;
      a.s[j].ld = in.ld;
      a.s[j].idx = in.idx;
      a.s[j].vals = in.vals;
      a.s[j].n_full = in.n_full;
      a.s[j].nseg = in.nseg;
      max_n = std::max(max_n, in.n);
    }
    if (stage == kTopkAll || stage == kTopkThreshold)
      hipLaunchKernelGGL(topk_sample_kernel, dim3(out_rows), dim3(kBig), 0, s, a);
    if (stage == kTopkAll) {
      const int64_t chunks = (max_n + kCompactChunk - 1) / kCompactChunk;
      if (chunks > 0)
        hipLaunchKernelGGL(topk_compact_kernel, dim3((unsigned)chunks, out_rows),
                           dim3(kCompactThreads), 0, s, a);
    }
    if (stage != kTopkThreshold)
      hipLaunchKernelGGL(topk_final_kernel, dim3(out_rows), dim3(kBig), 0, s, a);
    int32_t rc = hip_fail(hipGetLastError(), "topk launch");
    if (rc) return rc;
  }
  return FATHOM_OK;
}

}  // namespace fathom
