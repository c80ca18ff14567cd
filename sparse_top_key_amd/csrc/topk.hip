// Top-k key selection per decode step (explainer, problem statement: each
// generated token keeps the top k of the n scored keys).  Ranking: score
// descending, then index ascending; results are those of a full sort.
//
// Three launches per call (MI355X-first design; the pages give none):
//   topk_sample   one block per output row: reads a sample of the row
//                 (64-score runs spread evenly, about 16K scores; or a row of
//                 sampled logits) and picks a threshold key T expected to
//                 leave about 2.5k scores at or above it, by two 11-bit
//                 radix digits below the bits all sampled keys share.  Rows
//                 of at most 8192 scores take T = 0 (all).
//   topk_compact  the whole grid streams every row once and appends the
//                 (score key, index) words >= T to the row's candidate list
//                 (staged in LDS, one global atomic per block).
//   topk_final    one block per output row: if the candidates hold at least k
//                 and at most 8192 words they contain the exact top k (every
//                 score >= T is present).  The winners are ranked without a
//                 sort: words are bucketed on the 11 bits below their common
//                 prefix and each takes its bucket's offset plus the number of
//                 larger words in its bucket (a radix select plus a merge sort
//                 of in-wave bitonic runs when a bucket is too large).  Other
//                 rows are recomputed exactly: a 3-pass radix select over the
//                 whole row finds the k-th key, an index-ordered pass gathers
//                 the winners (ties at the k-th key by lowest index), and the
//                 same ranking orders them.
// The fused scan + top-k call reuses these kernels in stages: the threshold
// from sampled logits, a final over the candidate segments the scan wrote
// (rows out of range are flagged instead of recomputed), and an exact final
// for the flagged rows once their logits exist.
// Scores map to order-preserving uint32 keys after adding +0 (so -0 ranks as
// +0); a GQA group's score is its rows' fp32 scores added in fp64, in row
// order, rounded once.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kBig = 1024;            // threads of the per-row kernels
constexpr int kCompactThreads = 256;
constexpr int kCompactChunk = 16384;  // scores per compact block
constexpr int kRun = 64;              // contiguous scores per sample run
constexpr int kHistBins = 2048;
constexpr int kStage = 2048;           // candidates staged per compact block

struct TopkSess {
  const float *scores;
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
};

__device__ __forceinline__ float group_score(const float *__restrict__ row, int64_t ld,
                                             int group, int64_t i) {
  if (group == 1) return row[i];
  double acc = 0.0;
  for (int j = 0; j < group; ++j) acc = __dadd_rn(acc, (double)row[(int64_t)j * ld + i]);
  return (float)acc;
}

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
    int t = lane < kBig / 64 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int u = __shfl_up(t, off);
      if (lane >= off) t += u;
    }
    if (lane < kBig / 64) wave_tot[lane] = t;
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
__device__ uint64_t *sort_winners_desc(uint64_t *w, uint64_t *tmp, int m) {
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

__device__ void write_out(const TopkSess &S, int r, int k, const uint64_t *s, int m) {
  int32_t *idx = S.idx + (int64_t)r * k;
  float *vals = S.vals + (int64_t)r * k;
  for (int j = threadIdx.x; j < k; j += kBig) {
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
// spread evenly, about 16K in all; or all of a row of sampled logits), a
// threshold key T expected to leave about 2.5k of the row's n_full scores at
// or above it: the sample's keys are histogrammed on the 11 bits below their
// common prefix and T is the lower edge of the bin holding the rs-th
// largest.  Rows of at most 8192 scores take T = 0 (all).
__global__ __launch_bounds__(kBig) void topk_sample_kernel(TopkArgs a) {
  constexpr int kPer = (kSampleTarget + kRun + kBig - 1) / kBig;
  __shared__ int hist[kHistBins];
  __shared__ int wave_tot[16];
  __shared__ int s_res[2];
  __shared__ uint32_t red[48];
  const int o = blockIdx.x;
  const RowRef R = row_ref(a, o);
  const int64_t n = R.s->n, ld = R.s->ld, n_full = R.s->n_full;
  if (threadIdx.x == 0) {
    a.cnt[(int64_t)o * kCntStride] = 0;
    a.flag[o] = 0;
    a.redo[(o / a.rows_per_sess) * a.hkv + (o % a.rows_per_sess) / a.rows_per_kv] = 0;
  }
  if (n_full <= kCandCap) {
    if (threadIdx.x == 0) a.thr[o] = 0;
    return;
  }
  int64_t stride = (n * kRun + kSampleTarget - 1) / kSampleTarget;
  stride = (stride + kRun - 1) / kRun * kRun;
  if (stride < kRun) stride = kRun;
  const int runs = (int)((n + stride - 1) / stride);
  const int m = runs * kRun;
  // every load of the thread in flight at once (one row: plain loads first,
  // keys after)
  uint32_t v[kPer];
  uint32_t okm = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = threadIdx.x + j * kBig;
    const int64_t pos = (int64_t)(e / kRun) * stride + (e % kRun);
    okm |= (uint32_t)(e < m && pos < n) << j;
  }
  if (a.group == 1) {
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
  } else {
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
  // Two 11-bit digits below the bits all sampled keys share: T = the rs-th
  // largest key with its bits below the second digit cleared.
  const uint32_t diff = mx ^ mn;
  const int hb = diff ? 31 - __clz(diff) : 0;  // highest bit in which keys differ
  int sh = hb > 10 ? hb - 10 : 0;
  uint32_t prefix = sh + 11 >= 32 ? 0u : (mx >> (sh + 11)) << (sh + 11);
  uint32_t pmask = sh + 11 >= 32 ? 0u : ~((1u << (sh + 11)) - 1u);
  int rem = (int)rs;
  for (int pass = 0; pass < 2; ++pass) {
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
    for (int b = threadIdx.x; b < kHistBins; b += kBig) hist[b] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < m; j += kBig) {
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

// OR of v over the block.
__device__ uint64_t block_or64(uint64_t v, uint64_t *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v |= shfl_xor64(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = 0;
#pragma unroll
  for (int w = 0; w < kBig / 64; ++w) r |= red[w];
  __syncthreads();
  return r;
}

// Writes the kk largest of the unique words src[0..m) (1 <= kk <= m) to
// output row r in descending order, without sorting: words are bucketed by
// the 11 bits below their common prefix, the buckets at or above the one
// holding the kk-th word are laid out in descending bucket order, and each
// word's rank is its bucket's offset plus the number of larger words in its
// bucket.  Returns false, having written nothing, when one of those buckets
// holds more than kMaxBucket words (the caller then sorts).  Buckets grow
// when the candidates span two binades, so that the binning window starts in
// the exponent bits; a word's rank is a loop over its bucket, and even at 512
// words that costs far less than the sort it avoids.
constexpr int kMaxBucket = 512;

__device__ bool bucket_rank_out(const uint64_t *src, int m, int kk, uint64_t *buck, int *hist,
                                int *above, int *wave_tot, int *s_res, uint64_t *red,
                                const TopkSess &S, int r, int k) {
  const int t = threadIdx.x;
  uint64_t diff = 0;
  const uint64_t w0 = src[0];
  for (int j = t; j < m; j += kBig) diff |= src[j] ^ w0;
  diff = block_or64(diff, red);
  const int hb = diff ? 63 - __clzll(diff) : 0;  // highest bit in which words differ
  const int sh = hb > 10 ? hb - 10 : 0;
  for (int b = t; b < kHistBins; b += kBig) hist[b] = 0;
  if (t == 0) s_res[1] = 0;
  __syncthreads();
  for (int j = t; j < m; j += kBig) atomicAdd(&hist[(int)((src[j] >> sh) & (kHistBins - 1))], 1);
  __syncthreads();
  // above[d] = words in digits > d; thread t owns digits 2047-2t and 2046-2t
  const int d1 = kHistBins - 1 - 2 * t, d2 = d1 - 1;
  const int c1 = hist[d1], c2 = hist[d2];
  const int incl = block_inclusive_scan(c1 + c2, wave_tot);
  const int excl = incl - c1 - c2;
  above[d1] = excl;
  above[d2] = excl + c1;
  if (excl < kk && kk <= excl + c1) s_res[0] = d1;
  if (excl + c1 < kk && kk <= incl) s_res[0] = d2;
  __syncthreads();
  const int db = s_res[0];  // digit holding the kk-th word
  if ((d1 >= db && c1 > kMaxBucket) || (d2 >= db && c2 > kMaxBucket)) s_res[1] = 1;
  __syncthreads();
  if (s_res[1]) return false;
  // bucket order; above[d] becomes the end of bucket d
  for (int j = t; j < m; j += kBig) {
    const uint64_t w = src[j];
    const int d = (int)((w >> sh) & (kHistBins - 1));
    if (d >= db) buck[atomicAdd(&above[d], 1)] = w;
  }
  __syncthreads();
  const int total = above[db];
  int32_t *idx = S.idx + (int64_t)r * k;
  float *vals = S.vals + (int64_t)r * k;
  for (int p = t; p < total; p += kBig) {
    const uint64_t w = buck[p];
    const int d = (int)((w >> sh) & (kHistBins - 1));
    const int c = hist[d];
    const int b0 = above[d] - c;
    int rank = b0;
    for (int q = b0; q < b0 + c; ++q) rank += buck[q] > w;
    if (rank < kk) {
      idx[rank] = (int32_t)(~(uint32_t)w);
      vals[rank] = from_key((uint32_t)(w >> 32));
    }
  }
  for (int j = kk + t; j < k; j += kBig) {
    idx[j] = -1;
    vals[j] = -INFINITY;
  }
  return true;
}

// ---- exact selection of each row's top k -------------------------------------
__global__ __launch_bounds__(kBig) void topk_final_kernel(TopkArgs a) {
  __shared__ uint64_t s[kCandCap];
  __shared__ uint64_t win[FATHOM_MAX_K + kMaxBucket];
  __shared__ int hist[kHistBins];
  __shared__ int above[kHistBins];
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
  uint32_t cnt = 0;
  bool fused_over = false;
  if (a.stage == kTopkFusedFinal) {
    // the row's candidates sit in one segment per scan block
    const int nseg = S.nseg, seg_cap = kFusedCap / (nseg > 0 ? nseg : 1);
    const int c = threadIdx.x < nseg ? (int)a.seg_cnt[(int64_t)o * kMaxSeg + threadIdx.x] : 0;
    const int incl = block_inclusive_scan(c, wave_tot);
    s_off[threadIdx.x] = incl - c;
    if (threadIdx.x == kBig - 1) s_off[kMaxSeg] = incl;
    if (threadIdx.x == 0) s_res[1] = 0;
    __syncthreads();
    if (c > seg_cap) s_res[1] = 1;
    __syncthreads();
    cnt = (uint32_t)s_off[kMaxSeg];
    fused_over = s_res[1] != 0;
    __syncthreads();
  } else {
    cnt = a.cnt[(int64_t)o * kCntStride];
  }
  bool fast = !fused_over &&
              ((n <= kCandCap) || (cnt >= (uint32_t)k && cnt <= (uint32_t)kCandCap));
  if (a.stage == kTopkRedoFinal) {
    if (!a.flag[o]) return;  // this row was answered from its candidates
    fast = false;
  } else if (a.stage == kTopkFusedFinal && !fast) {
    // too few or too many candidates: the row is recomputed from full logits
    if (threadIdx.x == 0) {
      a.flag[o] = 1;
      a.redo[(o / a.rows_per_sess) * a.hkv + r / a.rows_per_kv] = 1;
    }
    return;
  }
  if (threadIdx.x == 0) s_count = 0;
  if (fast) {
    const int m = (int)cnt;
    if (a.stage == kTopkFusedFinal) {
      const int nseg = S.nseg, seg_cap = kFusedCap / (nseg > 0 ? nseg : 1);
      const uint64_t *fc = a.fcand + (int64_t)o * kFusedCap;
      // kBig / nseg threads per segment; each has 8 loads in flight before it
      // stores (segments hold at most seg_cap words: no overflow here)
      const int tps = kBig / (nseg > 0 ? nseg : 1);
      const int sg = threadIdx.x / tps, sub = threadIdx.x % tps;
      if (sg < nseg) {
        const int c = s_off[sg + 1] - s_off[sg];
        const uint64_t *src = fc + (int64_t)sg * seg_cap;
        uint64_t *dst = s + s_off[sg];
        for (int b0 = sub; b0 < c; b0 += 8 * tps) {
          uint64_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = b0 + u * tps;
            v[u] = src[i < c ? i : c - 1];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = b0 + u * tps;
            if (i < c) dst[i] = v[u];
          }
        }
      }
    } else {
      const uint64_t *cand = a.cand + (int64_t)o * kCandCap;
      for (int j = threadIdx.x; j < m; j += kBig) s[j] = cand[j];
    }
    __syncthreads();
    if (kk > 0 &&
        bucket_rank_out(s, m, kk, win, hist, above, wave_tot, s_res, red, S, r, k))
      return;
    if (kk > 0) {
      const uint64_t T = m > kk ? select_kth(s, m, kk, hist, wave_tot, s_res) : 0ull;
      for (int j = threadIdx.x; j < m; j += kBig)
        if (s[j] >= T) win[atomicAdd(&s_count, 1)] = s[j];
    }
  } else {
    // exact recomputation over the whole row
    int rem = kk;
    uint32_t prefix = 0, pmask = 0;
    const int shifts[3] = {21, 10, 0};
    const int bits[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass], nb = 1 << bits[pass];
      for (int b = threadIdx.x; b < kHistBins; b += kBig) hist[b] = 0;
      __syncthreads();
      for (int64_t i = threadIdx.x; i < n; i += kBig) {
        const uint32_t v = to_key(group_score(R.row, ld, a.group, i));
        if ((v & pmask) == prefix) atomicAdd(&hist[(v >> sh) & (nb - 1)], 1);
      }
      __syncthreads();
      int above = 0;
      const int d = find_digit(hist, nb, rem, &above, wave_tot, s_res);
      rem -= above;
      prefix |= (uint32_t)d << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
    }
    const uint32_t kth = prefix;  // key of the kk-th largest score
    const int need_eq = rem;      // how many scores equal to it are kept
    int eq_seen = 0;
    for (int64_t b0 = 0; b0 < n; b0 += (int64_t)kBig * 4) {
      uint32_t key[4];
      int eqc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = b0 + threadIdx.x * 4 + e;
        key[e] = i < n ? to_key(group_score(R.row, ld, a.group, i)) : 0u;
        eqc += (i < n && key[e] == kth);
      }
      const int incl = block_inclusive_scan(eqc, wave_tot);
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
        if (take) win[atomicAdd(&s_count, 1)] = compose(key[e], i);
      }
      eq_seen += wave_tot[kBig / 64 - 1];
      __syncthreads();
    }
  }
  __syncthreads();
  // win[0..kk) holds the winners
  if (!fast && kk > 0 &&
      bucket_rank_out(win, kk, kk, s, hist, above, wave_tot, s_res, red, S, r, k))
    return;
  const uint64_t *sorted = sort_winners_desc(win, s, kk);
  write_out(S, r, k, sorted, kk);
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
    int64_t max_n = 0;
    for (int j = 0; j < cnt; ++j) {
      const TopkSession &in = sess[s0 + j];
      a.s[j].scores = in.scores;
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
