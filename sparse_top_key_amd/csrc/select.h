// Per-row selection on one 1024-thread block, shared by the top-k kernels and
// the recompute step of the fused scan + top-k call (explainer, problem
// statement: each decode step keeps the top k of the n scored keys; ranking
// is score descending, then index ascending, as a full sort orders them).
// Scores map to order-preserving uint32 keys (to_key), candidates to 64-bit
// words (key, ~index); a GQA group's score is its rows' fp32 scores added in
// fp64 in row order, rounded once.  Every function is called by all threads
// of the block; LDS buffers are passed in by the caller.
#pragma once

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kSelThreads = 1024;  // threads of a selecting block
constexpr int kHistBins = 2048;    // radix digits of 11 bits
constexpr int kRankBins = 4096;    // ranking buckets (12 bits)

__device__ __forceinline__ float group_score(const float *__restrict__ row, int64_t ld,
                                             int group, int64_t i) {
  if (group == 1) return row[i];
  double acc = 0.0;
  for (int j = 0; j < group; ++j) acc = __dadd_rn(acc, (double)row[(int64_t)j * ld + i]);
  return (float)acc;
}

// Inclusive scan over the 1024 threads of a block (thread order).
__device__ int block_inclusive_scan(int v, int *wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int t = lane < kSelThreads / 64 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int u = __shfl_up(t, off);
      if (lane >= off) t += u;
    }
    if (lane < kSelThreads / 64) wave_tot[lane] = t;
  }
  __syncthreads();
  const int r = v + (wave > 0 ? wave_tot[wave - 1] : 0);
  __syncthreads();
  return r;
}

// Given hist[nbins] of the digits still in play, find digit d such that
// (#digits > d) < rem <= (#digits >= d).  Returns d; *above = #digits > d.
__device__ int find_digit(const int *hist, int nbins, int rem, int *above,
                          int *wave_tot, int *s_res) {
  // thread t owns digits hi = nbins-1-2t and hi-1 (descending order)
  const int t = threadIdx.x;
  const int d1 = nbins - 1 - 2 * t, d2 = d1 - 1;
  const int c1 = d1 >= 0 ? hist[d1] : 0;
  const int c2 = d2 >= 0 ? hist[d2] : 0;
  const int incl = block_inclusive_scan(c1 + c2, wave_tot);
  const int excl = incl - c1 - c2;
  if (excl < rem && rem <= incl) {
    if (excl + c1 >= rem) {
      s_res[0] = d1;
      s_res[1] = excl;
    } else {
      s_res[0] = d2;
      s_res[1] = excl + c1;
    }
  }
  __syncthreads();
  const int d = s_res[0];
  *above = s_res[1];
  __syncthreads();
  return d;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// In-wave bitonic sort of 128 words, descending: lane l holds elements 2l and
// 2l+1.  Stride 1 is a register compare; strides 2..64 exchange with the
// partner lane (distance stride/2).
__device__ __forceinline__ void wave_sort128_desc(uint64_t (&v)[2]) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 1) {
        const bool desc = ((2 * l) & size) == 0;
        if (desc ? (v[0] < v[1]) : (v[0] > v[1])) {
          const uint64_t x = v[0];
          v[0] = v[1];
          v[1] = x;
        }
        continue;
      }
      const int pt = stride >> 1;
      const uint64_t o0 = shfl_xor64(v[0], pt), o1 = shfl_xor64(v[1], pt);
      const uint64_t o[2] = {o0, o1};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = 2 * l + r;
        const bool lo = (e & stride) == 0;
        const bool desc = ((lo ? e : (e ^ stride)) & size) == 0;
        const bool keep_max = (lo == desc);
        const uint64_t mx = v[r] > o[r] ? v[r] : o[r], mn = v[r] > o[r] ? o[r] : v[r];
        v[r] = keep_max ? mx : mn;
      }
    }
  }
}

// Sort the m <= FATHOM_MAX_K = 2048 unique words w[0..m) descending, with
// entries past m read as 0; tmp is scratch of the same size.  Each wave
// sorts a run of 128 in registers, then merge-path rounds double the run
// length: thread t finds by binary search how many of the first 2t outputs
// of its pair of runs come from the first run, and writes outputs 2t, 2t+1.
// Returns the buffer holding the result.
__device__ __forceinline__ uint64_t *sort_winners_desc(uint64_t *w, uint64_t *tmp, int m) {
  int P = 128;
  while (P < m) P <<= 1;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  __syncthreads();
  if (wave < P / 128) {
    const int e0 = 128 * wave + 2 * lane;
    uint64_t v[2] = {e0 < m ? w[e0] : 0ull, e0 + 1 < m ? w[e0 + 1] : 0ull};
    wave_sort128_desc(v);
    w[e0] = v[0];
    w[e0 + 1] = v[1];
  }
  uint64_t *src = w, *dst = tmp;
  for (int L = 128; L < P; L <<= 1) {
    __syncthreads();
    if (t < P / 2) {
      const int base = (2 * t) / (2 * L) * (2 * L);
      const int d = 2 * t - base;
      const uint64_t *A = src + base, *B = src + base + L;
      int lo = d > L ? d - L : 0, hi = d < L ? d : L;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (A[mid] > B[d - 1 - mid])
          lo = mid + 1;
        else
          hi = mid;
      }
      int ia = lo, ib = d - lo;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const bool takeA = ib >= L || (ia < L && A[ia] > B[ib]);
        dst[base + d + r] = takeA ? A[ia++] : B[ib++];
      }
    }
    uint64_t *x = src;
    src = dst;
    dst = x;
  }
  __syncthreads();
  return src;
}

// Writes the first m of the words s (descending) as output row (idx, vals)
// of k entries, the rest as padding (-1, -inf).
__device__ void write_out(int32_t *idx, float *vals, int k, const uint64_t *s, int m) {
  for (int j = threadIdx.x; j < k; j += kSelThreads) {
    if (j < m) {
      const uint64_t c = s[j];
      idx[j] = (int32_t)(~(uint32_t)c);
      vals[j] = from_key((uint32_t)(c >> 32));
    } else {
      idx[j] = -1;
      vals[j] = -INFINITY;
    }
  }
}

// OR of v over the block.
__device__ uint64_t block_or64(uint64_t v, uint64_t *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v |= shfl_xor64(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) r |= red[w];
  __syncthreads();
  return r;
}

// Writes the kk largest of the unique words src[0..m) (1 <= kk <= m) to
// output row (idx, vals) in descending order, without sorting: words are
// bucketed by the 12 bits below their common prefix, the buckets at or above
// the one holding the kk-th word are laid out in descending bucket order, and
// each word's rank is its bucket's offset plus the number of larger words in
// its bucket.  Buckets grow when the candidates span two binades, so that the
// binning window starts in the exponent bits; a word's rank is a loop over
// its bucket, and even at 512 words that costs far less than a sort.  One
// larger bucket strictly above the kk-th word's (top keys clustered in a
// narrow score range: all of its words are winners, at most kk of them) is
// ranked on its own, binned again on the 11 bits below its own words' common
// prefix, in `sort_buf` (2 * FATHOM_MAX_K words; sorted there when that
// fails).  Returns false, having written nothing, for anything else (the
// caller then selects and sorts).  buck holds kBuckCap words, hist
// kRankBins ints, above kRankBins + 1.
// Words of b[b0 .. e) larger than w: 8 independent LDS reads per step (the
// last step's indices clamped to e - 1 and masked), so that a long bucket
// costs its reads' issue time rather than one LDS latency per word.
__device__ __forceinline__ int count_larger(const uint64_t *b, int b0, int e, uint64_t w) {
  int r = 0;
  for (int q = b0; q < e; q += 8) {
    uint64_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = b[q + u < e ? q + u : e - 1];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += (q + u < e) & (x[u] > w);
  }
  return r;
}

constexpr int kMaxBucket = 512;
constexpr int kBuckCap = FATHOM_MAX_K + kMaxBucket;

// PRE: the caller passes the bits in which the words differ (pre_diff) and
// has zeroed hist behind at least one block barrier.
template <bool PRE = false>
__device__ __forceinline__ bool bucket_rank_out(const uint64_t *src, int m, int kk, uint64_t *buck,
                                                int *hist, int *above,
                                                int *wave_tot, int *s_res, uint64_t *red,
                                                int32_t *idx, float *vals, int k,
                                                uint64_t *sort_buf, uint64_t pre_diff = 0) {
  const int t = threadIdx.x;
  uint64_t diff = pre_diff;
  if constexpr (!PRE) {
    const uint64_t w0 = src[0];
    for (int j = t; j < m; j += kSelThreads) diff |= src[j] ^ w0;
    diff = block_or64(diff, red);
  }
  const int hb = diff ? 63 - __clzll(diff) : 0;  // highest bit in which words differ
  const int sh = hb > 11 ? hb - 11 : 0;
  if (t == 0) s_res[1] = 0;
  if constexpr (!PRE) {
    for (int b = t; b < kRankBins; b += kSelThreads) hist[b] = 0;
    __syncthreads();
  }
  for (int j = t; j < m; j += kSelThreads)
    atomicAdd(&hist[(int)((src[j] >> sh) & (kRankBins - 1))], 1);
  __syncthreads();
  // above[d] = words in digits > d; thread t owns digits kRankBins-1-4t ..
  // kRankBins-4-4t (descending)
  constexpr int kOwn = kRankBins / kSelThreads;
  int cown[kOwn], sum = 0;
#pragma unroll
  for (int i = 0; i < kOwn; ++i) {
    cown[i] = hist[kRankBins - 1 - kOwn * t - i];
    sum += cown[i];
  }
  const int incl = block_inclusive_scan(sum, wave_tot);
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < kOwn; ++i) {
    const int d = kRankBins - 1 - kOwn * t - i;
    above[d] = run;
    if (run < kk && kk <= run + cown[i]) s_res[0] = d;
    run += cown[i];
  }
  __syncthreads();
  const int db = s_res[0];  // digit holding the kk-th word
  // big buckets at or above db: one strictly above db (all of its words are
  // winners) is ranked on its own; the kk-th word's bucket must stay small
#pragma unroll
  for (int i = 0; i < kOwn; ++i) {
    const int d = kRankBins - 1 - kOwn * t - i;
    if (d >= db && cown[i] > kMaxBucket) {
      atomicAdd(&s_res[1], d == db ? 2 : 1);
      if (d != db) above[kRankBins] = d;
    }
  }
  __syncthreads();
  const int nbig = s_res[1];
  if (nbig > 1) return false;
  const int dbig = nbig == 1 ? above[kRankBins] : -1;
  // bucket order; above[d] becomes the end of bucket d
  for (int j = t; j < m; j += kSelThreads) {
    const uint64_t w = src[j];
    const int d = (int)((w >> sh) & (kRankBins - 1));
    if (d >= db) buck[atomicAdd(&above[d], 1)] = w;
  }
  __syncthreads();
  const int total = above[db];
  for (int p = t; p < total; p += kSelThreads) {
    const uint64_t w = buck[p];
    const int d = (int)((w >> sh) & (kRankBins - 1));
    if (d == dbig) continue;
    const int c = hist[d];
    const int b0 = above[d] - c;
    const int rank = b0 + count_larger(buck, b0, b0 + c, w);
    if (rank < kk) {
      idx[rank] = (int32_t)(~(uint32_t)w);
      vals[rank] = from_key((uint32_t)(w >> 32));
    }
  }
  if (dbig >= 0) {
    // The big bucket (words buck[b0 .. b0+c), ranks b0 ..): binned again on
    // the 11 bits below its own words' common prefix and ranked within those
    // bins as above; should a bin still exceed the cap, the bucket is sorted.
    const int c = hist[dbig], b0 = above[dbig] - c;
    const uint64_t *bw = buck + b0;
    const int d1 = kHistBins - 1 - 2 * t, d2 = d1 - 1;  // digits of thread t (descending)
    uint64_t dif = 0;
    for (int j = t; j < c; j += kSelThreads) dif |= bw[j] ^ bw[0];
    dif = block_or64(dif, red);  // (its barrier also ends the ranking loop above)
    const int hb2 = dif ? 63 - __clzll(dif) : 0;
    const int sh2 = hb2 > 10 ? hb2 - 10 : 0;
    for (int b = t; b < kHistBins; b += kSelThreads) hist[b] = 0;
    if (t == 0) s_res[1] = 0;
    __syncthreads();
    for (int j = t; j < c; j += kSelThreads) atomicAdd(&hist[(int)((bw[j] >> sh2) & (kHistBins - 1))], 1);
    __syncthreads();
    const int h1 = hist[d1], h2 = hist[d2];
    const int inc2 = block_inclusive_scan(h1 + h2, wave_tot);
    above[d1] = inc2 - h1 - h2;
    above[d2] = inc2 - h2;
    if (h1 > kMaxBucket || h2 > kMaxBucket) s_res[1] = 1;
    __syncthreads();
    if (!s_res[1]) {
      for (int j = t; j < c; j += kSelThreads) {
        const uint64_t w = bw[j];
        sort_buf[atomicAdd(&above[(int)((w >> sh2) & (kHistBins - 1))], 1)] = w;
      }
      __syncthreads();
      for (int p = t; p < c; p += kSelThreads) {
        const uint64_t w = sort_buf[p];
        const int d = (int)((w >> sh2) & (kHistBins - 1));
        const int cnt = hist[d];
        const int s0 = above[d] - cnt;
        const int rank = b0 + s0 + count_larger(sort_buf, s0, s0 + cnt, w);
        idx[rank] = (int32_t)(~(uint32_t)w);
        vals[rank] = from_key((uint32_t)(w >> 32));
      }
    } else {
      for (int j = t; j < c; j += kSelThreads) sort_buf[j] = bw[j];
      const uint64_t *sorted = sort_winners_desc(sort_buf, sort_buf + FATHOM_MAX_K, c);
      for (int j = t; j < c; j += kSelThreads) {
        const uint64_t w = sorted[j];
        idx[b0 + j] = (int32_t)(~(uint32_t)w);
        vals[b0 + j] = from_key((uint32_t)(w >> 32));
      }
    }
  }
  for (int j = kk + t; j < k; j += kSelThreads) {
    idx[j] = -1;
    vals[j] = -INFINITY;
  }
  return true;
}

// LDS the exact row selection works in.
// Exact kk-th largest of the unique 64-bit words s[0..m) by 11-bit radix
// passes from the top bit; stops early once a whole digit bin is taken.
// Returns T such that exactly kk words are >= T.
__device__ uint64_t select_kth(const uint64_t *s, int m, int kk, int *hist, int *wave_tot,
                               int *s_res) {
  uint64_t prefix = 0, pmask = 0;
  int rem = kk;
  int hi = 64;
  while (hi > 0) {
    const int bits = hi >= 11 ? 11 : hi;
    const int sh = hi - bits;
    const int nb = 1 << bits;
    for (int b = threadIdx.x; b < kHistBins; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < m; j += kSelThreads) {
      const uint64_t v = s[j];
      if ((v & pmask) == prefix) atomicAdd(&hist[(int)((v >> sh) & (uint64_t)(nb - 1))], 1);
    }
    __syncthreads();
    int above = 0;
    const int d = find_digit(hist, nb, rem, &above, wave_tot, s_res);
    const int in_bin = hist[d];
    __syncthreads();
    rem -= above;
    prefix |= (uint64_t)d << sh;
    pmask |= (uint64_t)(nb - 1) << sh;
    hi = sh;
    if (in_bin == rem) break;  // the whole bin is kept: T = prefix, low bits 0
  }
  return prefix;
}

struct SelScratch {
  uint64_t *win;   // kBuckCap words: the winners
  uint64_t *s;     // kBuckCap + 2 * FATHOM_MAX_K words: buckets, sort space
  int *hist;       // kRankBins
  int *above;      // kRankBins + 1
  int *wave_tot;   // 16
  int *s_res;      // 2
  int *s_count;    // 1
  uint64_t *red;   // 16
};

// Exact top k of one row of n scores (row[i], or the fp64 sum of `group`
// rows ld apart) written to (idx, vals): a 3-pass radix select over the whole
// row finds the kk-th key, an index-ordered pass gathers the winners (ties at
// the kk-th key by lowest index), and they are ranked as above (sorted when
// that fails).
__device__ __forceinline__ void exact_row_topk(const float *row, int64_t ld, int group, int64_t n, int k,
                               int32_t *idx, float *vals, const SelScratch &X) {
  const int kk = (int)(n < k ? n : k);
  __syncthreads();  // the scratch may still be read by an earlier call
  if (threadIdx.x == 0) *X.s_count = 0;
  int rem = kk;
  uint32_t prefix = 0, pmask = 0;
  const int shifts[3] = {21, 10, 0};
  const int bits[3] = {11, 11, 10};
  for (int pass = 0; pass < 3 && kk > 0; ++pass) {
    const int sh = shifts[pass], nb = 1 << bits[pass];
    for (int b = threadIdx.x; b < kHistBins; b += kSelThreads) X.hist[b] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
      const uint32_t v = to_key(group_score(row, ld, group, i));
      if ((v & pmask) == prefix) atomicAdd(&X.hist[(v >> sh) & (nb - 1)], 1);
    }
    __syncthreads();
    int above = 0;
    const int d = find_digit(X.hist, nb, rem, &above, X.wave_tot, X.s_res);
    rem -= above;
    prefix |= (uint32_t)d << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
  }
  const uint32_t kth = prefix;  // key of the kk-th largest score
  const int need_eq = rem;      // how many scores equal to it are kept
  int eq_seen = 0;
  for (int64_t b0 = 0; kk > 0 && b0 < n; b0 += (int64_t)kSelThreads * 4) {
    uint32_t key[4];
    int eqc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = b0 + threadIdx.x * 4 + e;
      key[e] = i < n ? to_key(group_score(row, ld, group, i)) : 0u;
      eqc += (i < n && key[e] == kth);
    }
    const int incl = block_inclusive_scan(eqc, X.wave_tot);
    int rank = eq_seen + incl - eqc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = b0 + threadIdx.x * 4 + e;
      if (i >= n) continue;
      bool take = key[e] > kth;
      if (key[e] == kth) {
        take = rank < need_eq;
        ++rank;
      }
      if (take) X.win[atomicAdd(X.s_count, 1)] = compose(key[e], i);
    }
    eq_seen += X.wave_tot[kSelThreads / 64 - 1];
    __syncthreads();
  }
  __syncthreads();
  // X.win[0..kk) holds the winners
  if (kk > 0 && bucket_rank_out(X.win, kk, kk, X.s, X.hist, X.above, X.wave_tot, X.s_res, X.red,
                                idx, vals, k, X.s + kBuckCap))
    return;
  const uint64_t *sorted = sort_winners_desc(X.win, X.s, kk);
  write_out(idx, vals, k, sorted, kk);
}

// LDS of the fused final (fused_final_row): the row's candidate words (the
// ranking also uses their upper part as sort space), the winners, ranking
// bins, reduction slots and the segments' offsets.
struct FinalScratch {
  uint64_t *s;      // kCandCap
  uint64_t *win;    // kBuckCap
  int *hist;        // kRankBins
  int *above;       // kRankBins + 1
  uint64_t *red;    // kSelThreads / 64
  int *wave_tot;    // 16
  int *s_res;       // 2
  int *s_count;     // 1
  int *s_off;       // kMaxSeg + 1
};
constexpr int64_t kFinalScratchBytes =
    (int64_t)(kCandCap + kBuckCap + kSelThreads / 64) * 8 +
    (int64_t)(2 * kRankBins + 1 + 16 + 2 + 1 + kMaxSeg + 1) * 4;

// Exact top k of one output row of a fused scan + top-k call, from the
// candidate words the candidate scan stored: min(c_b, seg_cap) words in each
// of the nseg segments of frow (seg_cap = kFusedCap / nseg words apart), the
// rest of every block's count c_b in the overflow list ov (*ov_cnt words).  Every score at
// or above the row's threshold is a candidate, so when the row holds k to
// kCandCap of them (or n <= kCandCap: all keys) they contain its top k,
// which are ranked and written; otherwise nothing is written and false is
// returned (the row needs its full logits).
__device__ __forceinline__ bool fused_final_row(const uint64_t *frow, const uint32_t *segc, int nseg,
                                                const uint64_t *ov, const uint32_t *ov_cnt, int64_t n,
                                                int k, int32_t *idx, float *vals,
                                                const FinalScratch &X) {
  const int kk = (int)(n < k ? n : k);
  // the ranking histogram is cleared while the loads below are in flight
  for (int b = threadIdx.x; b < kRankBins; b += kSelThreads) X.hist[b] = 0;
  // kSelThreads / nseg threads per segment; each loads the first kSpec of its
  // words before the segment counts are known, so that both reads share one
  // memory latency (words past a segment's count are dropped; segments hold
  // at most seg_cap words)
  constexpr int kSpec = 8;
  const int seg_cap = kFusedCap / (nseg > 0 ? nseg : 1);
  const int tps = kSelThreads / (nseg > 0 ? nseg : 1);
  const int sg = threadIdx.x / tps, sub = threadIdx.x % tps;
  const uint64_t *fseg = frow + (int64_t)sg * seg_cap;
  uint64_t spec[kSpec];
  if (sg < nseg) {
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const int i = sub + u * tps;
      spec[u] = fseg[i < seg_cap ? i : seg_cap - 1];
    }
  }
  // the row's count: min(c, seg_cap) words in each segment, plus the
  // overflow list's count (the rest of every block's count)
  const int c = threadIdx.x < nseg ? (int)segc[threadIdx.x] : 0;
  const uint32_t ovf = *ov_cnt;
  const int kept = c < seg_cap ? c : seg_cap;
  const int incl = block_inclusive_scan(kept, X.wave_tot);
  X.s_off[threadIdx.x] = incl - kept;
  if (threadIdx.x == kSelThreads - 1) X.s_off[kMaxSeg] = incl;
  if (threadIdx.x == 0) *X.s_count = 0;
  __syncthreads();
  const int stored = X.s_off[kMaxSeg];
  const uint32_t cnt = (uint32_t)stored + ovf;
  if (!(n <= kCandCap || (cnt >= (uint32_t)k && cnt <= (uint32_t)kCandCap))) return false;
  const int m = (int)cnt;
  // the words loaded ahead, then the rest of each segment with 8 loads in
  // flight per thread before it stores; each thread keeps the OR and the AND
  // of the words it stores (the bits in which the row's words differ)
  uint64_t w_or = 0, w_and = ~0ull;
  if (sg < nseg) {
    const int cs = (sg + 1 < nseg ? X.s_off[sg + 1] : X.s_off[kMaxSeg]) - X.s_off[sg];
    uint64_t *dst = X.s + X.s_off[sg];
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const int i = sub + u * tps;
      if (i < cs) {
        dst[i] = spec[u];
        w_or |= spec[u];
        w_and &= spec[u];
      }
    }
    for (int b0 = sub + kSpec * tps; b0 < cs; b0 += 8 * tps) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = b0 + u * tps;
        v[u] = fseg[i < cs ? i : cs - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = b0 + u * tps;
        if (i < cs) {
          dst[i] = v[u];
          w_or |= v[u];
          w_and &= v[u];
        }
      }
    }
  }
  // then the overflow list (m <= kCandCap words in all)
  for (int j = threadIdx.x; j < m - stored; j += kSelThreads) {
    const uint64_t w = ov[j];
    X.s[stored + j] = w;
    w_or |= w;
    w_and &= w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    w_or |= shfl_xor64(w_or, off);
    w_and &= shfl_xor64(w_and, off);
  }
  if ((threadIdx.x & 63) == 0) {
    X.red[threadIdx.x >> 6] = w_or;
    X.win[threadIdx.x >> 6] = w_and;  // (win is free until the ranking places words)
  }
  __syncthreads();
  uint64_t diff = 0;
  if (kk > 0) {
    uint64_t o = 0, a = ~0ull;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      o |= X.red[w];
      a &= X.win[w];
    }
    diff = o & ~a;
  }
  if (kk > 0 && bucket_rank_out<true>(X.s, m, kk, X.win, X.hist, X.above, X.wave_tot, X.s_res,
                                      X.red, idx, vals, k, X.s + kBuckCap, diff))
    return true;
  if (kk > 0) {
    const uint64_t T = m > kk ? select_kth(X.s, m, kk, X.hist, X.wave_tot, X.s_res) : 0ull;
    for (int j = threadIdx.x; j < m; j += kSelThreads)
      if (X.s[j] >= T) X.win[atomicAdd(X.s_count, 1)] = X.s[j];
  }
  __syncthreads();
  // win[0..kk) holds the winners
  const uint64_t *sorted = sort_winners_desc(X.win, X.s, kk);
  write_out(idx, vals, k, sorted, kk);
  return true;
}

}  // namespace
}  // namespace fathom
