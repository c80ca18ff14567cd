/*
 * fathom_oracle.c -- plain, slow, single-threaded CPU definition of Fathom's
 * read path: pack (4-bit per-channel quantisation into channel-major bit
 * planes), plan (reverse water-filling of a per-query bit budget), scan
 * (approximate logits from the top t_c planes of each channel) and top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the bench's CPU-baseline leg and the
 * smoke check load it.  It shares no code, header or table with the HIP path.
 *
 * Sources (all on the pages about "Fathom: Per-Query Read Depth for Sparse
 * Decoding over Offloaded KV Caches", arXiv 2609.17652):
 *   [EXP]  the Chinese explainer (papers.ananclaw.com), sections
 *          "核心方法" (core method: storage side / read side) and
 *          "关键伪代码" (key pseudocode), "反向注水 vs 固定预算" (intuition).
 *   [SUM]  the proomt.com summary, "Summary" bullet list.
 * Points the pages leave open are resolved as listed in the design notes
 * (readings R1..R14); each function below names the readings it relies on.
 *
 * Floating point: compiled with -O2 -fno-fast-math -ffp-contract=off, so every
 * float/double operation below is one IEEE-754 round-to-nearest operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* Words per plane row: the plane of one (kv head, channel) holds one bit per
 * key, 32 keys per little-endian uint32 word, padded to a multiple of 2048
 * keys (64 words).  Layout reading R1/R2. */
int64_t orc_plane_words(int64_t n) { return 64 * ((n + 2047) / 2048); }

/* ------------------------------------------------------------------------ */
/* Pack.  [EXP] core method, storage side: K is quantised to 4 bits per
 * channel, stored channel-major, and each channel's 4 bits are split into
 * bit planes, plane t=0 holding the least significant bit and t=3 the most
 * significant.  Readings:
 *   R2  quantiser = 16 equal cells between the channel's min and max over the
 *       n keys, code = floor((x - lo) / delta), delta = (hi - lo) / 16,
 *       clamped to 15 (x == hi lands in the top cell);
 *   R4  a constant channel (hi == lo) gives delta = 0 and every code 0;
 *   R1  plane slot s = 3 - p, so the most significant plane comes first and
 *       the first t slots of a channel are its top t planes;
 *   R5  sigma^2 = population variance of the stored (dequantised) 4-bit
 *       values, computed exactly from integer code sums.
 * keys: fp32 element (token i, kv head h, channel c) at
 *       keys[i*stride_tok + h*stride_head + c].
 * codes  [hkv][d][n]  (uint8, may be NULL)
 * planes [hkv][d][4][W]
 * lo, hi, sigma2 [hkv][d]                                                    */
int orc_pack(const float *keys, int64_t n, int hkv, int d, int64_t stride_tok,
             int64_t stride_head, uint8_t *codes, uint32_t *planes, float *lo,
             float *hi, float *sigma2) {
  if (!keys || !planes || !lo || !hi || !sigma2 || n < 1 || hkv < 1 || d < 1)
    return ORC_BAD;
  const int64_t W = orc_plane_words(n);
  memset(planes, 0, (size_t)hkv * d * 4 * W * sizeof(uint32_t));
  for (int h = 0; h < hkv; ++h) {
    for (int c = 0; c < d; ++c) {
      const float *col = keys + (int64_t)h * stride_head + c;
      /* channel range over all keys */
      float mn = col[0], mx = col[0];
      for (int64_t i = 1; i < n; ++i) {
        float x = col[i * stride_tok];
        if (x < mn) mn = x;
        if (x > mx) mx = x;
      }
      /* R4: -0 and +0 are one key value; the stored range ends are +0. */
      mn = mn + 0.0f;
      mx = mx + 0.0f;
      float range = mx - mn;
      float delta = range * 0.0625f; /* exact: scaling by 2^-4 */
      int64_t s1 = 0, s2 = 0;
      uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
      for (int64_t i = 0; i < n; ++i) {
        float x = col[i * stride_tok];
        int code = 0;
        if (delta != 0.0f) {
          float u = x - mn;
          float y = u / delta;
          double fl = floor((double)y);
          code = fl > 15.0 ? 15 : (int)fl;
        }
        if (codes) codes[((int64_t)h * d + c) * n + i] = (uint8_t)code;
        s1 += code;
        s2 += (int64_t)code * code;
        for (int p = 0; p < 4; ++p) {
          if ((code >> p) & 1) {
            int slot = 3 - p;
            pl[slot * W + i / 32] |= 1u << (i % 32);
          }
        }
      }
      /* Var(code) = (n*S2 - S1^2) / n^2, exact in int64 for n <= 2^26;
       * Var(dequantised) = Var(code) * delta^2 (dequantisation is affine). */
      int64_t num = n * s2 - s1 * s1;
      double var_code = (double)num / ((double)n * (double)n);
      double dd = (double)delta * (double)delta;
      double var = var_code * dd;
      lo[h * d + c] = mn;
      hi[h * d + c] = mx;
      sigma2[h * d + c] = (float)var;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Plan.  [EXP] core method, read side, and the key pseudocode: each query
 * has a budget of B bits per key; channel importance is the key-channel
 * variance weighted by the query (R6: w_c = (q_c*q_c)*sigma_c^2 in fp32,
 * multiply then multiply, no fused multiply-add); the budget fills channels
 * up to the 4-bit cap in descending w (R8: equal w puts the lower channel
 * index first; R7: fill-to-cap), so with that order the first B / 4
 * channels get 4 bits, the next one B % 4, and the rest none.
 * R9: 0 <= B <= 4d.
 * q [hq][d] fp32, sigma2 [hkv][d], budget [hq], plan out [hq][d] uint8.
 * Query head h uses kv head h / (hq / hkv) (R12).                          */
typedef struct {
  float w;
  int c;
} orc_wc;

static int orc_cmp_w_desc(const void *a, const void *b) {
  const orc_wc *x = (const orc_wc *)a, *y = (const orc_wc *)b;
  if (x->w > y->w) return -1;
  if (x->w < y->w) return 1;
  return (x->c < y->c) ? -1 : (x->c > y->c);
}

int orc_plan(const float *q, int hq, int hkv, int d, const float *sigma2,
             const int32_t *budget, uint8_t *plan) {
  if (!q || !sigma2 || !budget || !plan || hq < 1 || hkv < 1 || hq % hkv)
    return ORC_BAD;
  const int G = hq / hkv;
  orc_wc *order = (orc_wc *)malloc(sizeof(orc_wc) * d);
  if (!order) return ORC_BAD;
  for (int h = 0; h < hq; ++h) {
    int B = budget[h];
    if (B < 0 || B > 4 * d) {
      free(order);
      return ORC_BAD;
    }
    const float *sg = sigma2 + (int64_t)(h / G) * d;
    for (int c = 0; c < d; ++c) {
      float qq = q[(int64_t)h * d + c] * q[(int64_t)h * d + c];
      order[c].w = qq * sg[c];
      order[c].c = c;
    }
    qsort(order, d, sizeof(orc_wc), orc_cmp_w_desc);
    /* the budget fills channels to the 4-bit cap in that order: the first
       B / 4 channels are read in full, the next one gets the remaining
       B % 4 bits, every later channel none */
    const int full = B / 4, part = B % 4;
    for (int j = 0; j < d; ++j) {
      uint8_t t = 0;
      if (j < full) t = 4;
      else if (j == full) t = (uint8_t)part;
      plan[(int64_t)h * d + order[j].c] = t;
    }
  }
  free(order);
  return ORC_OK;
}

/* Fixed-width baseline plan (the pages' 136-bit scans read the r = 32 channels
 * with the largest |q_c| in full; R10): channels ordered by |q_c| descending,
 * ties to the lower index, the first r get all 4 planes, the rest none. */
int orc_plan_fixed(const float *q, int hq, int d, int r, uint8_t *plan) {
  if (!q || !plan || hq < 1 || r < 0 || r > d) return ORC_BAD;
  orc_wc *order = (orc_wc *)malloc(sizeof(orc_wc) * d);
  if (!order) return ORC_BAD;
  for (int h = 0; h < hq; ++h) {
    for (int c = 0; c < d; ++c) {
      order[c].w = fabsf(q[(int64_t)h * d + c]);
      order[c].c = c;
    }
    qsort(order, d, sizeof(orc_wc), orc_cmp_w_desc);
    for (int j = 0; j < d; ++j)
      plan[(int64_t)h * d + order[j].c] = (uint8_t)(j < r ? 4 : 0);
  }
  free(order);
  return ORC_OK;
}

/* Rate-distortion variant of the water-filling.  [EXP] key pseudocode notes
 * that the original treats the allocation more finely than fill-to-cap and
 * gives no table; [EXP] "反向注水 vs 固定预算" says that with close channel
 * importances the budget spreads almost evenly.  Reading R16: each read bit
 * of channel c at depth t (t = 0..3 bits already read) lowers the channel's
 * distortion w_c * 4^-t by a gain proportional to w_c * 4^-t, and the budget
 * buys the B largest gains (gain desc, then channel asc, then t asc).  A
 * channel's gains fall with t, so the bits taken from a channel are always
 * its top ones, and t_c = the number of its gains taken.  Gains are compared
 * exactly in fp64 (w_c * 2^(-2t) is exact there).
 * Same arguments and w_c as orc_plan.                                       */
typedef struct {
  double g;
  int c, t;
} orc_gain;

static int orc_cmp_gain(const void *a, const void *b) {
  const orc_gain *x = (const orc_gain *)a, *y = (const orc_gain *)b;
  if (x->g > y->g) return -1;
  if (x->g < y->g) return 1;
  if (x->c != y->c) return x->c < y->c ? -1 : 1;
  return (x->t < y->t) ? -1 : (x->t > y->t);
}

int orc_plan_rd(const float *q, int hq, int hkv, int d, const float *sigma2,
                const int32_t *budget, uint8_t *plan) {
  if (!q || !sigma2 || !budget || !plan || hq < 1 || hkv < 1 || hq % hkv)
    return ORC_BAD;
  const int G = hq / hkv;
  orc_gain *gains = (orc_gain *)malloc(sizeof(orc_gain) * 4 * d);
  if (!gains) return ORC_BAD;
  for (int h = 0; h < hq; ++h) {
    int B = budget[h];
    if (B < 0 || B > 4 * d) {
      free(gains);
      return ORC_BAD;
    }
    const float *sg = sigma2 + (int64_t)(h / G) * d;
    for (int c = 0; c < d; ++c) {
      float qq = q[(int64_t)h * d + c] * q[(int64_t)h * d + c];
      float w = qq * sg[c];
      for (int t = 0; t < 4; ++t) {
        gains[4 * c + t].g = ldexp((double)w, -2 * t);
        gains[4 * c + t].c = c;
        gains[4 * c + t].t = t;
      }
    }
    qsort(gains, (size_t)4 * d, sizeof(orc_gain), orc_cmp_gain);
    for (int c = 0; c < d; ++c) plan[(int64_t)h * d + c] = 0;
    for (int j = 0; j < B; ++j) plan[(int64_t)h * d + gains[j].c] += 1;
  }
  free(gains);
  return ORC_OK;
}

/* One plan per GQA group.  [EXP] "反向注水 vs 固定预算" lists sharing the
 * channel importance across a GQA group as a direction (the pages decide per
 * head).  Reading R17: the group's importance of channel c is
 * sigma_c^2 * sum over the group's heads of q_hc^2, the squares added in fp32
 * in head order and the product rounded once (fp32); the fill-to-cap walk of
 * orc_plan spends budget[g] on it, and every head of the group gets that plan,
 * so the group reads exactly budget[g] bits per key.
 * budget [hkv] (one per kv head), plan out [hq][d].                          */
int orc_plan_group(const float *q, int hq, int hkv, int d, const float *sigma2,
                   const int32_t *budget, uint8_t *plan) {
  if (!q || !sigma2 || !budget || !plan || hq < 1 || hkv < 1 || hq % hkv)
    return ORC_BAD;
  const int G = hq / hkv;
  orc_wc *order = (orc_wc *)malloc(sizeof(orc_wc) * d);
  if (!order) return ORC_BAD;
  for (int g = 0; g < hkv; ++g) {
    int B = budget[g];
    if (B < 0 || B > 4 * d) {
      free(order);
      return ORC_BAD;
    }
    for (int c = 0; c < d; ++c) {
      float sq = 0.0f;
      for (int j = 0; j < G; ++j) {
        float qc = q[(int64_t)(g * G + j) * d + c];
        sq = sq + qc * qc;
      }
      order[c].w = sq * sigma2[(int64_t)g * d + c];
      order[c].c = c;
    }
    qsort(order, d, sizeof(orc_wc), orc_cmp_w_desc);
    /* fill to the 4-bit cap in that order, as orc_plan: B / 4 channels in
       full, the next one B % 4 bits, the rest none; one plan for all heads */
    const int full = B / 4, part = B % 4;
    for (int j = 0; j < d; ++j) {
      const uint8_t t = j < full ? 4 : (j == full ? (uint8_t)part : 0);
      for (int k = 0; k < G; ++k) plan[(int64_t)(g * G + k) * d + order[j].c] = t;
    }
  }
  free(order);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The 4-bit code of key i in channel c of kv head h, rebuilt bit by bit from
 * the planes (slot 3 - p holds bit p). */
static int orc_code_from_planes(const uint32_t *planes, int64_t W, int d, int h,
                                int c, int64_t i) {
  const uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
  int code = 0;
  for (int p = 0; p < 4; ++p) {
    uint32_t word = pl[(3 - p) * W + i / 32];
    code |= (int)((word >> (i % 32)) & 1u) << p;
  }
  return code;
}

/* The value a query reads from the top t planes of a code: the t-bit prefix
 * floor(code / 2^(4-t)) (0 when t = 0).  [EXP] core method: the first t
 * planes of a channel are that channel's t-bit quantiser. */
static int orc_prefix(int code, int t) { return t == 0 ? 0 : code >> (4 - t); }

/* The side stream of the fixed-width baselines (R10), value of key i of kv
 * head g: 8 bits: meta [hkv][n], one byte per key; 4 bits (the r = 16 form,
 * whose metadata is r/4 bits per key): meta [hkv][ceil(n/2)], two keys per
 * byte, key i in the low nibble of byte i/2 when i is even, the high nibble
 * when it is odd. */
static double orc_meta(const uint8_t *meta, int bits, int g, int64_t n, int64_t i) {
  if (bits == 8) return (double)meta[(int64_t)g * n + i];
  const uint8_t b = meta[(int64_t)g * ((n + 1) / 2) + i / 2];
  return (double)((b >> (4 * (i & 1))) & 15);
}

/* Score of key i for query head h.  [EXP] core method, read side: the query
 * reads, per channel, only the planes its plan gives that channel.  Reading
 * R11: the unread low bits sit at their midpoint, i.e. the t-bit prefix r is
 * reconstructed at the centre of its cell of width delta*2^(4-t):
 *     deq_t = lo + (r + 1/2) * delta * 2^(4-t)       (t = 0: lo + 8*delta),
 *     s_i   = sum_c q_c * deq_{t_c}(code_ic)  [+ meta_scale * meta_i],
 * evaluated in fp64 (rounded once to fp32 by the callers). */
static double orc_score(const uint32_t *planes, int64_t W, const float *lo, const float *hi,
                        int64_t n, int d, int g, const float *qh, const uint8_t *ph,
                        const uint8_t *meta, int bits, float meta_scale, int64_t i) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) {
    int t = ph[c];
    float l = lo[g * d + c], u = hi[g * d + c];
    float delta = (u - l) * 0.0625f;
    int r = orc_prefix(orc_code_from_planes(planes, W, d, g, c, i), t);
    double cell = (double)delta * (double)(1 << (4 - t));
    double deq = (double)l + ((double)r + 0.5) * cell;
    s += (double)qh[c] * deq;
  }
  if (meta) s += (double)meta_scale * orc_meta(meta, bits, g, n, i);
  return s;
}

static int orc_scan_bits(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
                         int hkv, int d, const float *q, const uint8_t *plan, int hq,
                         const uint8_t *meta, int bits, float meta_scale, float *logits,
                         int64_t ld) {
  if (!planes || !lo || !hi || !q || !plan || !logits || n < 0 || hkv < 1 ||
      hq % hkv || ld < n)
    return ORC_BAD;
  const int G = hq / hkv;
  const int64_t W = orc_plane_words(n);
  for (int h = 0; h < hq; ++h)
    for (int64_t i = 0; i < n; ++i)
      logits[(int64_t)h * ld + i] =
          (float)orc_score(planes, W, lo, hi, n, d, h / G, q + (int64_t)h * d,
                           plan + (int64_t)h * d, meta, bits, meta_scale, i);
  return ORC_OK;
}

static int orc_scan_at_bits(const uint32_t *planes, const float *lo, const float *hi,
                            int64_t n, int hkv, int d, const float *q, const uint8_t *plan,
                            int hq, const uint8_t *meta, int bits, float meta_scale,
                            const int64_t *keys, int64_t nk, float *out) {
  if (!planes || !lo || !hi || !q || !plan || !keys || !out || hkv < 1 ||
      hq % hkv)
    return ORC_BAD;
  const int G = hq / hkv;
  const int64_t W = orc_plane_words(n);
  for (int h = 0; h < hq; ++h)
    for (int64_t j = 0; j < nk; ++j) {
      const int64_t i = keys[j];
      if (i < 0 || i >= n) return ORC_BAD;
      out[(int64_t)h * nk + j] =
          (float)orc_score(planes, W, lo, hi, n, d, h / G, q + (int64_t)h * d,
                           plan + (int64_t)h * d, meta, bits, meta_scale, i);
    }
  return ORC_OK;
}

/* Scan: every key's score (orc_score) for every query head, logits [hq][ld];
 * meta: the optional 8-bit side stream [hkv][n]. */
int orc_scan(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
             int hkv, int d, const float *q, const uint8_t *plan, int hq,
             const uint8_t *meta, float meta_scale, float *logits, int64_t ld) {
  return orc_scan_bits(planes, lo, hi, n, hkv, d, q, plan, hq, meta, 8, meta_scale, logits,
                       ld);
}

/* The same scores at chosen keys only: out[h][j] = s_{keys[j]} of head h
 * (for spot checks of large layers). */
int orc_scan_at(const uint32_t *planes, const float *lo, const float *hi,
                int64_t n, int hkv, int d, const float *q, const uint8_t *plan,
                int hq, const uint8_t *meta, float meta_scale,
                const int64_t *keys, int64_t nk, float *out) {
  return orc_scan_at_bits(planes, lo, hi, n, hkv, d, q, plan, hq, meta, 8, meta_scale, keys,
                          nk, out);
}

/* orc_scan and orc_scan_at with the 4-bit side stream (meta [hkv][ceil(n/2)],
 * see orc_meta). */
int orc_scan_meta4(const uint32_t *planes, const float *lo, const float *hi, int64_t n,
                   int hkv, int d, const float *q, const uint8_t *plan, int hq,
                   const uint8_t *meta, float meta_scale, float *logits, int64_t ld) {
  return orc_scan_bits(planes, lo, hi, n, hkv, d, q, plan, hq, meta, 4, meta_scale, logits,
                       ld);
}

int orc_scan_at_meta4(const uint32_t *planes, const float *lo, const float *hi,
                      int64_t n, int hkv, int d, const float *q, const uint8_t *plan,
                      int hq, const uint8_t *meta, float meta_scale,
                      const int64_t *keys, int64_t nk, float *out) {
  return orc_scan_at_bits(planes, lo, hi, n, hkv, d, q, plan, hq, meta, 4, meta_scale, keys,
                          nk, out);
}

/* The plane reads themselves: out[h][i][c] = t_c-bit prefix of code_ic. */
int orc_read_prefixes(const uint32_t *planes, int64_t n, int hkv, int d,
                      const uint8_t *plan, int hq, uint8_t *out) {
  if (!planes || !plan || !out || hkv < 1 || hq % hkv) return ORC_BAD;
  const int G = hq / hkv;
  const int64_t W = orc_plane_words(n);
  for (int h = 0; h < hq; ++h)
    for (int64_t i = 0; i < n; ++i)
      for (int c = 0; c < d; ++c)
        out[((int64_t)h * n + i) * d + c] = (uint8_t)orc_prefix(
            orc_code_from_planes(planes, W, d, h / G, c, i),
            plan[(int64_t)h * d + c]);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-k.  [EXP] problem statement: every generated token scores the n keys
 * and keeps the top k.  Reading R13: keys are ranked by (score descending,
 * index ascending); rows shorter than k are padded with index -1 and score
 * -inf.  Reading R12: for a GQA group of G query heads the group score of key
 * i is the sum of the G rows' fp32 scores, added in row order in fp64 and
 * rounded once to fp32.
 * scores [rows][ld]; idx, vals [rows/group][k]. */
typedef struct {
  float s;
  int32_t i;
} orc_si;

static int orc_cmp_score(const void *a, const void *b) {
  const orc_si *x = (const orc_si *)a, *y = (const orc_si *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->i < y->i) ? -1 : (x->i > y->i);
}

int orc_topk(const float *scores, int rows, int64_t n, int64_t ld, int group,
             int k, int32_t *idx, float *vals) {
  if (!scores || !idx || !vals || rows < 1 || group < 1 || rows % group ||
      k < 1 || n < 0 || ld < n || n > 2147483647)
    return ORC_BAD;
  orc_si *all = (orc_si *)malloc(sizeof(orc_si) * (size_t)(n > 0 ? n : 1));
  if (!all) return ORC_BAD;
  for (int o = 0; o < rows / group; ++o) {
    for (int64_t i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int r = 0; r < group; ++r)
        acc += (double)scores[(int64_t)(o * group + r) * ld + i];
      all[i].s = (float)acc;
      all[i].i = (int32_t)i;
    }
    qsort(all, (size_t)n, sizeof(orc_si), orc_cmp_score);
    for (int j = 0; j < k; ++j) {
      if (j < n) {
        idx[(int64_t)o * k + j] = all[j].i;
        vals[(int64_t)o * k + j] = all[j].s;
      } else {
        idx[(int64_t)o * k + j] = -1;
        vals[(int64_t)o * k + j] = -INFINITY;
      }
    }
  }
  free(all);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Sparse decode attention over the selected keys.  [EXP] problem statement:
 * every generated token runs attention over the top k of the n keys the scan
 * kept; "与 V 端稀疏化互补" and the future-work list: V stays dense.  The
 * pages give no layout for this step.  Reading R19: full-precision K and V
 * rows of the selected keys (token-major, fp16 widened exactly to fp32 by the
 * caller of this function), softmax over the selected keys only:
 *   s_i = scale * sum_c q_c K_ic,  m = max s_i,  p_i = exp(s_i - m),
 *   out_c = sum_i p_i V_ic / sum_i p_i,  lse = m + log(sum_i p_i),
 * all in fp64 and rounded once to fp32.  Entries of idx below 0 are skipped
 * (the padding of short rows); an entry listed twice counts twice.  A row
 * with no entry gives out = 0 and lse = -inf.
 * q [hq][d]; K, V element (token i, kv head g, channel c) at
 * [i*stride_tok + g*stride_head + c]; idx [hq/group][k] (row o serves query
 * heads o*group .. o*group+group-1, which share one kv head);
 * out [hq][d], lse [hq].                                                    */
int orc_sparse_attention(const float *q, int hq, int hkv, int d, const float *K,
                         const float *V, int64_t n, int64_t stride_tok,
                         int64_t stride_head, const int32_t *idx, int group, int k,
                         float scale, float *out, float *lse) {
  if (!q || !K || !V || !idx || !out || !lse || hq < 1 || hkv < 1 || d < 1 ||
      hq % hkv || group < 1 || (hq / hkv) % group || k < 0 || n < 0)
    return ORC_BAD;
  const int G = hq / hkv;
  double *s = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  double *acc = (double *)malloc(sizeof(double) * (size_t)d);
  if (!s || !acc) {
    free(s);
    free(acc);
    return ORC_BAD;
  }
  for (int o = 0; o < hq / group; ++o) {
    const int32_t *row = idx + (int64_t)o * k;
    for (int j = 0; j < k; ++j)
      if (row[j] >= n) {
        free(s);
        free(acc);
        return ORC_BAD;
      }
    for (int r = 0; r < group; ++r) {
      const int h = o * group + r, g = h / G;
      double m = -INFINITY;
      for (int j = 0; j < k; ++j) {
        if (row[j] < 0) continue;
        const float *kr = K + (int64_t)row[j] * stride_tok + (int64_t)g * stride_head;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += (double)q[(int64_t)h * d + c] * (double)kr[c];
        s[j] = (double)scale * dot;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int c = 0; c < d; ++c) acc[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        if (row[j] < 0) continue;
        const double p = exp(s[j] - m);
        const float *vr = V + (int64_t)row[j] * stride_tok + (int64_t)g * stride_head;
        l += p;
        for (int c = 0; c < d; ++c) acc[c] += p * (double)vr[c];
      }
      for (int c = 0; c < d; ++c) out[(int64_t)h * d + c] = l > 0.0 ? (float)(acc[c] / l) : 0.0f;
      lse[h] = l > 0.0 ? (float)(m + log(l)) : -INFINITY;
    }
  }
  free(s);
  free(acc);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Append keys to a packed layer.  [EXP] deployment warnings, item 3: when the
 * upstream 4-bit K is re-quantised nothing else has to be rebuilt, since the
 * planes are that K; the stored 4-bit K is reused per token (关键实验与数据,
 * storage cost).  Reading R20: a decode step's new keys are quantised with
 * the layer's stored range, code = floor((x - lo) / delta) with the fp32
 * subtract and divide of R2, clamped to 0..15; values outside [lo, hi] are
 * counted.  delta == 0 gives code 0.  sigma^2 stays the stored estimate.  Bits of the tokens n_old ..
 * n_old + m - 1 are set in plane rows of W words (W >= orc_plane_words of
 * n_old + m); every other bit is left as it was.
 * keys: element (new token j, kv head h, channel c) at
 * keys[j*stride_tok + h*stride_head + c]; planes [hkv][d][4][W].
 * Returns the number of clamped values through *clamped.                   */
int orc_append(const float *keys, int64_t m, int hkv, int d, int64_t stride_tok,
               int64_t stride_head, int64_t n_old, uint32_t *planes, int64_t W,
               const float *lo, const float *hi, int64_t *clamped) {
  if (!planes || !lo || !hi || !clamped || m < 0 || n_old < 0 || hkv < 1 || d < 1 ||
      (m > 0 && !keys) || W < orc_plane_words(n_old + m))
    return ORC_BAD;
  int64_t count = 0;
  for (int h = 0; h < hkv; ++h) {
    for (int c = 0; c < d; ++c) {
      const float l = lo[h * d + c], u = hi[h * d + c];
      const float delta = (u - l) * 0.0625f;
      uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
      for (int64_t j = 0; j < m; ++j) {
        const float x = keys[j * stride_tok + (int64_t)h * stride_head + c];
        int code = 0;
        if (delta != 0.0f) {
          const float y = (x - l) / delta;
          const double fl = floor((double)y);
          code = fl < 0.0 ? 0 : (fl > 15.0 ? 15 : (int)fl);
        }
        count += (x < l || x > u);
        const int64_t i = n_old + j;
        for (int s = 0; s < 4; ++s) {
          const uint32_t bit = (uint32_t)((code >> (3 - s)) & 1);
          uint32_t *word = pl + (int64_t)s * W + i / 32;
          *word = (*word & ~(1u << (i % 32))) | (bit << (i % 32));
        }
      }
    }
  }
  *clamped = count;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-block ranges.  [EXP] deployment warnings, item 3 (the planes are the
 * stored 4-bit K; re-quantising it must not force anything else to be
 * rebuilt) and the problem statement (long sessions that grow by a token per
 * decode step).  Reading R22: the range (lo, hi) of a channel is kept per
 * block of ORC_RB = 2048 consecutive keys instead of per layer, so a session
 * whose key ranges drift quantises its later blocks with ranges of their own
 * and no stored code is ever re-quantised.
 *   pack:   each block's range is the min and max of its own keys (R2 and R4
 *           within the block: delta_b = (hi_b - lo_b) / 16, codes clamped to
 *           15, -0 stored as +0); planes as orc_pack.
 *   sigma2: the pooled within-block variance of the dequantised values,
 *           sum over blocks in block order of fp64(var_b * (n_b / n)), var_b
 *           = fp64(fp64((n_b S2_b - S1_b^2) / (n_b n_b)) * delta_b^2) exactly
 *           as R5 computes it for one block, rounded once to fp32 (so a layer
 *           of one block has R5's sigma2).
 *   scan:   key i of block b = i / ORC_RB reads lo_b, delta_b in the formula
 *           of orc_scan.
 *   append: a block that holds no key before the call takes, per (kv head,
 *           channel), the range of the block before it widened to cover the
 *           keys the call puts in it (block 0: those keys' own min and max);
 *           a block that already holds keys keeps its range, and keys outside
 *           it are clamped and counted as in orc_append.
 * lo, hi: [hkv][nbc][d] (block-major: the d ranges of one block are
 * contiguous), nbc >= the number of blocks (a capacity).                    */
#define ORC_RB 2048

int64_t orc_range_blocks(int64_t n) { return (n + ORC_RB - 1) / ORC_RB; }

/* index of (kv head h, channel c, block b) in lo / hi */
static int64_t orc_rix(int h, int c, int64_t b, int64_t nbc, int d) {
  return ((int64_t)h * nbc + b) * d + c;
}

static int orc_quantise(float x, float l, float delta) {
  if (delta == 0.0f) return 0;
  const double fl = floor((double)((x - l) / delta));
  return fl < 0.0 ? 0 : (fl > 15.0 ? 15 : (int)fl);
}

int orc_pack_blocked(const float *keys, int64_t n, int hkv, int d, int64_t stride_tok,
                     int64_t stride_head, uint32_t *planes, float *lo, float *hi,
                     int64_t nbc, float *sigma2) {
  const int64_t nb = orc_range_blocks(n);
  if (!keys || !planes || !lo || !hi || !sigma2 || n < 1 || hkv < 1 || d < 1 || nbc < nb)
    return ORC_BAD;
  const int64_t W = orc_plane_words(n);
  memset(planes, 0, (size_t)hkv * d * 4 * W * sizeof(uint32_t));
  for (int h = 0; h < hkv; ++h) {
    for (int c = 0; c < d; ++c) {
      const float *col = keys + (int64_t)h * stride_head + c;
      uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
      double acc = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        const int64_t i0 = b * ORC_RB, i1 = i0 + ORC_RB < n ? i0 + ORC_RB : n;
        float mn = col[i0 * stride_tok], mx = mn;
        for (int64_t i = i0 + 1; i < i1; ++i) {
          const float x = col[i * stride_tok];
          if (x < mn) mn = x;
          if (x > mx) mx = x;
        }
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        const float delta = (mx - mn) * 0.0625f;
        lo[orc_rix(h, c, b, nbc, d)] = mn;
        hi[orc_rix(h, c, b, nbc, d)] = mx;
        int64_t s1 = 0, s2 = 0;
        for (int64_t i = i0; i < i1; ++i) {
          const int code = orc_quantise(col[i * stride_tok], mn, delta);
          s1 += code;
          s2 += (int64_t)code * code;
          for (int p = 0; p < 4; ++p)
            if ((code >> p) & 1) pl[(3 - p) * W + i / 32] |= 1u << (i % 32);
        }
        const int64_t nn = i1 - i0;
        const double var_code = (double)(nn * s2 - s1 * s1) / ((double)nn * (double)nn);
        const double var = var_code * ((double)delta * (double)delta);
        acc += var * ((double)nn / (double)n);
      }
      sigma2[h * d + c] = (float)acc;
    }
  }
  return ORC_OK;
}

static double orc_score_blocked(const uint32_t *planes, int64_t W, const float *lo,
                                const float *hi, int64_t nbc, int d, int g, const float *qh,
                                const uint8_t *ph, int64_t i) {
  const int64_t b = i / ORC_RB;
  double s = 0.0;
  for (int c = 0; c < d; ++c) {
    const int t = ph[c];
    const float l = lo[orc_rix(g, c, b, nbc, d)], u = hi[orc_rix(g, c, b, nbc, d)];
    const float delta = (u - l) * 0.0625f;
    const int r = orc_prefix(orc_code_from_planes(planes, W, d, g, c, i), t);
    const double cell = (double)delta * (double)(1 << (4 - t));
    s += (double)qh[c] * ((double)l + ((double)r + 0.5) * cell);
  }
  return s;
}

int orc_scan_blocked(const uint32_t *planes, const float *lo, const float *hi, int64_t nbc,
                     int64_t n, int hkv, int d, const float *q, const uint8_t *plan, int hq,
                     float *logits, int64_t ld) {
  if (!planes || !lo || !hi || !q || !plan || !logits || n < 0 || hkv < 1 || hq % hkv ||
      ld < n || nbc < orc_range_blocks(n))
    return ORC_BAD;
  const int G = hq / hkv;
  const int64_t W = orc_plane_words(n);
  for (int h = 0; h < hq; ++h)
    for (int64_t i = 0; i < n; ++i)
      logits[(int64_t)h * ld + i] = (float)orc_score_blocked(
          planes, W, lo, hi, nbc, d, h / G, q + (int64_t)h * d, plan + (int64_t)h * d, i);
  return ORC_OK;
}

int orc_scan_blocked_at(const uint32_t *planes, const float *lo, const float *hi, int64_t nbc,
                        int64_t n, int hkv, int d, const float *q, const uint8_t *plan, int hq,
                        const int64_t *keys, int64_t nk, float *out) {
  if (!planes || !lo || !hi || !q || !plan || !keys || !out || hkv < 1 || hq % hkv ||
      nbc < orc_range_blocks(n))
    return ORC_BAD;
  const int G = hq / hkv;
  const int64_t W = orc_plane_words(n);
  for (int h = 0; h < hq; ++h)
    for (int64_t j = 0; j < nk; ++j) {
      if (keys[j] < 0 || keys[j] >= n) return ORC_BAD;
      out[(int64_t)h * nk + j] = (float)orc_score_blocked(
          planes, W, lo, hi, nbc, d, h / G, q + (int64_t)h * d, plan + (int64_t)h * d, keys[j]);
    }
  return ORC_OK;
}

int orc_append_blocked(const float *keys, int64_t m, int hkv, int d, int64_t stride_tok,
                       int64_t stride_head, int64_t n_old, uint32_t *planes, int64_t W,
                       float *lo, float *hi, int64_t nbc, int64_t *clamped) {
  if (!planes || !lo || !hi || !clamped || m < 0 || n_old < 0 || hkv < 1 || d < 1 ||
      (m > 0 && !keys) || W < orc_plane_words(n_old + m) ||
      nbc < orc_range_blocks(n_old + m))
    return ORC_BAD;
  int64_t count = 0;
  const int64_t first_new = orc_range_blocks(n_old);  /* blocks with no key yet */
  const int64_t nb_end = orc_range_blocks(n_old + m);
  for (int h = 0; h < hkv; ++h) {
    for (int c = 0; c < d; ++c) {
      /* ranges of the blocks this call starts, in block order */
      for (int64_t b = first_new; b < nb_end; ++b) {
        const int64_t i0 = b * ORC_RB, i1 = i0 + ORC_RB < n_old + m ? i0 + ORC_RB : n_old + m;
        float mn, mx;
        if (b > 0) {
          mn = lo[orc_rix(h, c, b - 1, nbc, d)];
          mx = hi[orc_rix(h, c, b - 1, nbc, d)];
        } else {
          mn = mx = keys[(i0 - n_old) * stride_tok + (int64_t)h * stride_head + c];
        }
        for (int64_t i = i0; i < i1; ++i) {
          const float x = keys[(i - n_old) * stride_tok + (int64_t)h * stride_head + c];
          if (x < mn) mn = x;
          if (x > mx) mx = x;
        }
        lo[orc_rix(h, c, b, nbc, d)] = mn + 0.0f;
        hi[orc_rix(h, c, b, nbc, d)] = mx + 0.0f;
      }
      uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
      for (int64_t j = 0; j < m; ++j) {
        const int64_t i = n_old + j, b = i / ORC_RB;
        const float l = lo[orc_rix(h, c, b, nbc, d)], u = hi[orc_rix(h, c, b, nbc, d)];
        const float x = keys[j * stride_tok + (int64_t)h * stride_head + c];
        const int code = orc_quantise(x, l, (u - l) * 0.0625f);
        count += (x < l || x > u);
        for (int s = 0; s < 4; ++s) {
          const uint32_t bit = (uint32_t)((code >> (3 - s)) & 1);
          uint32_t *word = pl + (int64_t)s * W + i / 32;
          *word = (*word & ~(1u << (i % 32))) | (bit << (i % 32));
        }
      }
    }
  }
  *clamped = count;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-channel code histograms.  hist[h][c][v] = number of keys i < n whose
 * 4-bit code in channel c of kv head h is v, read back bit by bit from the
 * planes (rows of W words).                                                 */
int orc_code_hist(const uint32_t *planes, int64_t n, int hkv, int d, int64_t W,
                  uint32_t *hist) {
  if (!planes || !hist || n < 0 || hkv < 1 || d < 1 || W < orc_plane_words(n)) return ORC_BAD;
  for (int h = 0; h < hkv; ++h)
    for (int c = 0; c < d; ++c) {
      uint32_t *hc = hist + ((int64_t)h * d + c) * 16;
      const uint32_t *pl = planes + ((int64_t)h * d + c) * 4 * W;
      for (int v = 0; v < 16; ++v) hc[v] = 0;
      for (int64_t i = 0; i < n; ++i) {
        int code = 0;
        for (int s = 0; s < 4; ++s) code = (code << 1) | (int)((pl[s * W + i / 32] >> (i % 32)) & 1u);
        hc[code] += 1;
      }
    }
  return ORC_OK;
}

/* Calibrated allocation.  [EXP] key pseudocode: the original allocates more
 * finely than fill-to-cap without saying how; the intuition section ties the
 * allocation to how much each channel's error moves the logit.  Reading R21:
 * reading channel c to depth t leaves, per key, the gap between its 4-bit
 * value and the t-bit cell centre (R11); over the layer's keys that error is
 * E_c(t) * delta_c^2 with
 *     E_c(t) = sum_v hist_c[v] * ((v mod 2^(4-t)) + 1/2 - 2^(3-t))^2
 * (exact in fp64: counts times quarter-integers), and it enters query head
 * h's logit with weight q_hc^2.  The plan minimises
 *     sum_c cost_hc(t_c),  cost_hc(t) = fl64(fl64(q_hc^2 * delta_c^2) * E_c(t))
 * (q_hc^2 and delta_c^2 exact in fp64) over all plans with sum t_c = B,
 * 0 <= t_c <= 4, by dynamic programming over the channels in order:
 *     F_0 = [0, inf, ...];  F_{c+1}[b] = min_t F_c[b - t] + cost_hc(t)
 * (one fp64 add each; t tried in increasing order, a later t replaces the
 * best only when strictly smaller), then the choices are followed back from
 * F_d[B].  delta_c = fl32(fl32(hi - lo) * 1/16) as in R2.
 * hist [hkv][d][16]; budget [hq]; plan out [hq][d].                         */
/* E_c(t) of R21 for every (kv head, channel) and t = 0..4, in delta^2 units:
 * E out [hkv][d][5].                                                        */
int orc_depth_errors(const uint32_t *hist, int hkv, int d, double *E) {
  if (!hist || !E || hkv < 1 || d < 1) return ORC_BAD;
  for (int64_t hc = 0; hc < (int64_t)hkv * d; ++hc)
    for (int t = 0; t <= 4; ++t) {
      const int m = 1 << (4 - t);
      double e = 0.0;
      for (int v = 0; v < 16; ++v) {
        const double off = (double)(v % m) + 0.5 - 0.5 * m;
        e += (double)hist[hc * 16 + v] * (off * off);
      }
      E[hc * 5 + t] = e;
    }
  return ORC_OK;
}

int orc_plan_calibrated(const float *q, int hq, int hkv, int d, const float *lo,
                        const float *hi, const uint32_t *hist, const int32_t *budget,
                        uint8_t *plan) {
  if (!q || !lo || !hi || !hist || !budget || !plan || hq < 1 || hkv < 1 || hq % hkv || d < 1)
    return ORC_BAD;
  const int G = hq / hkv;
  double *cost = (double *)malloc(sizeof(double) * 5 * d);
  double *E = (double *)malloc(sizeof(double) * 5 * d * hkv);
  double *F = (double *)malloc(sizeof(double) * (4 * d + 1));
  double *Fn = (double *)malloc(sizeof(double) * (4 * d + 1));
  uint8_t *choice = (uint8_t *)malloc((size_t)d * (4 * d + 1));
  int rc = ORC_OK;
  if (!cost || !E || !F || !Fn || !choice || orc_depth_errors(hist, hkv, d, E) != ORC_OK) {
    rc = ORC_BAD;
    goto done;
  }
  for (int h = 0; h < hq; ++h) {
    const int B = budget[h];
    if (B < 0 || B > 4 * d) {
      rc = ORC_BAD;
      goto done;
    }
    const int g = h / G;
    for (int c = 0; c < d; ++c) {
      const float delta = (hi[g * d + c] - lo[g * d + c]) * 0.0625f;
      const double qd = (double)q[(int64_t)h * d + c] * (double)q[(int64_t)h * d + c] *
                        ((double)delta * (double)delta);
      for (int t = 0; t <= 4; ++t) cost[c * 5 + t] = qd * E[((int64_t)g * d + c) * 5 + t];
    }
    for (int b = 0; b <= B; ++b) F[b] = b == 0 ? 0.0 : INFINITY;
    for (int c = 0; c < d; ++c) {
      for (int b = 0; b <= B; ++b) {
        double best = INFINITY;
        int bt = 0;
        for (int t = 0; t <= 4 && t <= b; ++t) {
          const double v = F[b - t] + cost[c * 5 + t];
          if (v < best) {
            best = v;
            bt = t;
          }
        }
        Fn[b] = best;
        choice[(int64_t)c * (4 * d + 1) + b] = (uint8_t)bt;
      }
      for (int b = 0; b <= B; ++b) F[b] = Fn[b];
    }
    int b = B;
    for (int c = d - 1; c >= 0; --c) {
      const int t = choice[(int64_t)c * (4 * d + 1) + b];
      plan[(int64_t)h * d + c] = (uint8_t)t;
      b -= t;
    }
  }
done:
  free(cost);
  free(E);
  free(F);
  free(Fn);
  free(choice);
  return rc;
}

/* One calibrated plan per GQA group (readings R17 and R21 together): the
 * group's weight of channel c is S_c * delta_c^2, S_c = the fp64 sum in head
 * order of the squares q_hc^2 (each exact in fp64, and so is their sum), the
 * cost of depth t is fl64(fl64(S_c * delta_c^2) * E_c(t)), and the same DP
 * spends budget[g] (one per kv head); every head of the group gets the row.
 * A group of one head gives exactly orc_plan_calibrated.
 * budget [hkv]; plan out [hq][d].                                           */
int orc_plan_calibrated_group(const float *q, int hq, int hkv, int d, const float *lo,
                              const float *hi, const uint32_t *hist, const int32_t *budget,
                              uint8_t *plan) {
  if (!q || !lo || !hi || !hist || !budget || !plan || hq < 1 || hkv < 1 || hq % hkv || d < 1)
    return ORC_BAD;
  const int G = hq / hkv;
  double *E = (double *)malloc(sizeof(double) * 5 * d * hkv);
  double *cost = (double *)malloc(sizeof(double) * 5 * d);
  double *F = (double *)malloc(sizeof(double) * (4 * d + 1));
  double *Fn = (double *)malloc(sizeof(double) * (4 * d + 1));
  uint8_t *choice = (uint8_t *)malloc((size_t)d * (4 * d + 1));
  int rc = ORC_OK;
  if (!E || !cost || !F || !Fn || !choice || orc_depth_errors(hist, hkv, d, E) != ORC_OK) {
    rc = ORC_BAD;
    goto done;
  }
  for (int g = 0; g < hkv; ++g) {
    const int B = budget[g];
    if (B < 0 || B > 4 * d) {
      rc = ORC_BAD;
      goto done;
    }
    for (int c = 0; c < d; ++c) {
      const float delta = (hi[g * d + c] - lo[g * d + c]) * 0.0625f;
      double S = 0.0;
      for (int j = 0; j < G; ++j) {
        const double qc = (double)q[(int64_t)(g * G + j) * d + c];
        S = S + qc * qc;
      }
      const double wd = S * ((double)delta * (double)delta);
      for (int t = 0; t <= 4; ++t) cost[c * 5 + t] = wd * E[((int64_t)g * d + c) * 5 + t];
    }
    for (int b = 0; b <= B; ++b) F[b] = b == 0 ? 0.0 : INFINITY;
    for (int c = 0; c < d; ++c) {
      for (int b = 0; b <= B; ++b) {
        double best = INFINITY;
        int bt = 0;
        for (int t = 0; t <= 4 && t <= b; ++t) {
          const double v = F[b - t] + cost[c * 5 + t];
          if (v < best) {
            best = v;
            bt = t;
          }
        }
        Fn[b] = best;
        choice[(int64_t)c * (4 * d + 1) + b] = (uint8_t)bt;
      }
      for (int b = 0; b <= B; ++b) F[b] = Fn[b];
    }
    int b = B;
    for (int c = d - 1; c >= 0; --c) {
      const int t = choice[(int64_t)c * (4 * d + 1) + b];
      for (int j = 0; j < G; ++j) plan[(int64_t)(g * G + j) * d + c] = (uint8_t)t;
      b -= t;
    }
  }
done:
  free(E);
  free(cost);
  free(F);
  free(Fn);
  free(choice);
  return rc;
}
