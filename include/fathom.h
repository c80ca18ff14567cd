/*
 * fathom.h -- C ABI of the MI355X (gfx950) implementation of Fathom's read
 * path over a 4-bit, channel-major, bit-plane K cache:
 *
 *     fathom_pack -> fathom_plan -> fathom_scan -> fathom_topk
 *                                  (-> fathom_sparse_attention)
 *
 * The method is the one described on the pages about "Fathom: Per-Query Read
 * Depth for Sparse Decoding over Offloaded KV Caches" (arXiv 2609.17652);
 * citations below name the Chinese explainer page (papers.ananclaw.com) and
 * its section headings.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Plain C: pointers, sizes, an opaque stream.  `stream` is a hipStream_t
 *    (NULL = the default stream).  Every GPU call only enqueues work on that
 *    stream; nothing synchronises inside the library.
 *  - Ownership: the caller allocates and frees every buffer (inputs, outputs,
 *    workspaces).  The library never allocates, frees or keeps pointers; the
 *    one exception is the static device array of fathom_topk_noalloc.
 *  - Device pointers are HBM pointers unless an argument says it may also be
 *    pinned host memory (allocated with hipHostMalloc, e.g. torch's
 *    pin_memory); such memory is read zero-copy over the host link.
 *  - Return value: FATHOM_OK, or an error code.  Argument errors are detected
 *    on the host before anything is enqueued; fathom_last_error() then holds
 *    a one-line, thread-local description.  Faults during execution surface
 *    on the stream as HIP errors, like any kernel's.
 *  - Shapes: d (head dimension) must be 128 (FATHOM_ERR_UNSUPPORTED
 *    otherwise).  Query head h of a layer reads kv head h / (hq / hkv)
 *    (grouped-query attention); hq must be a multiple of hkv.
 *  - Inputs must be finite (no NaN/Inf keys, queries or scores); behaviour on
 *    non-finite inputs is unspecified.
 *  - Thread safety: calls are reentrant; two calls that write the same
 *    buffers must be ordered by the caller (same stream or events).
 */
#ifndef FATHOM_H
#define FATHOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FATHOM_ABI_VERSION 2
#define FATHOM_HEAD_DIM 128
#define FATHOM_MAX_K 2048         /* largest k accepted by the top-k calls */
#define FATHOM_MAX_SESSIONS 64    /* sessions per batched call */
#define FATHOM_MAX_ATTN_K (1 << 20) /* selected keys per row of sparse attention */

enum {
  FATHOM_OK = 0,
  FATHOM_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad budget, ...   */
  FATHOM_ERR_UNSUPPORTED = 2, /* valid but not implemented (d != 128, ...) */
  FATHOM_ERR_HIP = 3,         /* a HIP runtime call or launch failed        */
  FATHOM_ERR_WORKSPACE = 4    /* workspace missing or smaller than needed   */
};

enum { FATHOM_F16 = 0, FATHOM_F32 = 1 }; /* key element types */

int32_t fathom_abi_version(void);
const char *fathom_last_error(void);

/* ---- sizes -------------------------------------------------------------- */

/* Words per plane row: one bit per key, 32 keys per uint32 word, padded to a
 * whole number of 2048-key blocks: W = 64 * ceil(n / 2048). */
int64_t fathom_plane_words(int64_t n);
/* Bytes of the plane array of one layer: hkv * d * 4 * W * 4. */
int64_t fathom_planes_bytes(int64_t n, int32_t hkv, int32_t d);
/* Workspace bytes fathom_pack needs for n keys (0 on bad arguments). */
int64_t fathom_pack_workspace_bytes(int64_t n, int32_t hkv, int32_t d);
/* Workspace bytes fathom_topk needs for `out_rows` = rows / group output rows
 * (independent of n).  fathom_topk_batched needs this for the sum of its
 * sessions' output rows. */
int64_t fathom_topk_workspace_bytes(int32_t out_rows, int32_t k);

/* ---- pack (storage side) -------------------------------------------------
 * Explainer, section 核心方法 (core method), storage side: K is quantised to
 * 4 bits per channel and stored channel-major, each channel's 4 bits split
 * into bit planes; the first t planes of a channel are its t-bit quantiser.
 *
 * keys      device, token-major: element (token i, kv head h, channel c) at
 *           keys[i*stride_tok + h*stride_head + c] (strides in elements,
 *           channel stride 1), dtype FATHOM_F16 or FATHOM_F32, n >= 1.
 * planes    device (HBM) output, uint32[hkv][d][4][W]: slot s of channel c
 *           holds bit (3 - s) of the codes, so slot 0 is the most significant
 *           plane and the top t planes of a channel are the t*W contiguous
 *           words starting at slot 0.  Bit j of word w belongs to key 32w + j;
 *           padding bits (keys >= n) are 0.
 * lo, hi    device outputs fp32[hkv][d]: the channel's minimum and maximum
 *           over the n keys.  delta = (hi - lo) * 1/16 (fp32), code =
 *           min(15, floor((x - lo) / delta)) with IEEE fp32 subtract and
 *           divide; delta == 0 gives code 0.
 * sigma2    device output fp32[hkv][d]: variance of the dequantised 4-bit
 *           values lo + (code + 1/2) delta, computed exactly from integer code
 *           sums: fp32((n*S2 - S1^2) / n^2 * delta^2) in fp64.
 * ws        device workspace of at least fathom_pack_workspace_bytes bytes.
 * Enqueues 4 kernels.  Outputs are bit-identical to the CPU definition.    */
int32_t fathom_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                    int32_t d, int64_t stride_tok, int64_t stride_head,
                    uint32_t *planes, float *lo, float *hi, float *sigma2,
                    void *ws, int64_t ws_bytes, void *stream);

/* ---- plan (read side) ----------------------------------------------------
 * Explainer, sections 核心方法 (read side) and 关键伪代码: each query head
 * spends a budget of B bits per key over channels by reverse water-filling:
 * importance w_c = (q_c * q_c) * sigma2_c (fp32, two rounded multiplies),
 * channels visited by w descending (equal w: lower channel first), each
 * taking min(4, remaining budget) bits.  Channels may get 0 bits.
 *
 * q            device fp32[hq][d]
 * sigma2       device fp32[hkv][d] (from fathom_pack or any non-negative
 *              calibrated variance)
 * budget_bits  HOST int32[hq], each in [0, 4d] (else FATHOM_ERR_INVALID_ARG)
 * plan         device output uint8[hq][d]: t_c in 0..4, sum_c t_c = B.     */
int32_t fathom_plan(const float *q, int32_t hq, int32_t hkv, int32_t d,
                    const float *sigma2, const int32_t *budget_bits,
                    uint8_t *plan, void *stream);

/* Rate-distortion variant of the allocation.  The explainer's key-pseudocode
 * section notes that the original allocates more finely than fill-to-cap,
 * and its intuition section (反向注水 vs 固定预算) that close importances
 * spread the budget; neither gives the rule, so this one is a reading: a
 * channel read to depth t keeps an error term proportional to w_c * 4^-t
 * (one more plane quarters the quantisation cell), reading bit t+1 gains in
 * proportion to w_c * 4^-t, and the B largest gains are bought (ties: lower
 * channel, then shallower bit), which minimises sum_c w_c * 4^-t_c over all
 * plans with sum t_c = B, 0 <= t_c <= 4.  Gains are compared exactly (fp64).
 * Same w_c, arguments, ownership and errors as fathom_plan; q and sigma2
 * must be finite.  Output t_c in 0..4 with sum_c t_c = B.                  */
int32_t fathom_plan_rd(const float *q, int32_t hq, int32_t hkv, int32_t d,
                       const float *sigma2, const int32_t *budget_bits,
                       uint8_t *plan, void *stream);

/* One plan per GQA group.  The explainer's intuition section lists sharing
 * the channel importance across a GQA group as a direction (the pages plan
 * per head).  Group g (query heads g*G .. g*G+G-1, G = hq / hkv) uses
 * W_c = fp32(sigma2_gc * S_c), S_c = the fp32 sum in head order of the
 * rounded squares q_hc * q_hc, and the fill-to-cap walk of fathom_plan with
 * budget_bits[g]; every head of the group receives that row, so the group's
 * scan reads exactly budget_bits[g] plane bits per key.
 * budget_bits  HOST int32[hkv], each in [0, 4d] (else FATHOM_ERR_INVALID_ARG)
 * plan         device output uint8[hq][d] (G equal rows per group).
 * Other arguments as for fathom_plan.                                       */
int32_t fathom_plan_group(const float *q, int32_t hq, int32_t hkv, int32_t d,
                          const float *sigma2, const int32_t *budget_bits,
                          uint8_t *plan, void *stream);

/* Calibrated allocation (two calls).  The explainer's key-pseudocode section
 * says the original allocates more finely than fill-to-cap without giving
 * the rule; this is a stated reading that measures each channel's error on
 * the layer itself.
 *
 * fathom_code_hist: hist[h][c][v] = number of keys i < n whose 4-bit code in
 * channel c of kv head h is v (v = 0..15), read from the planes.
 *   planes  device or pinned-host, 16-byte aligned, rows of plane_words
 *           words (0: fathom_plane_words(n)); bits of keys >= n are ignored
 *   hist    device output uint32[hkv][d][16]
 *
 * fathom_plan_calibrated: reading channel c to depth t leaves each key the
 * gap between its 4-bit value and its t-bit cell centre; over the layer that
 * is delta_c^2 * E_c(t), E_c(t) = sum_v hist_c[v] * (v mod 2^(4-t) + 1/2 -
 * 2^(3-t))^2 (exact in fp64), and it moves head h's logit with weight
 * q_hc^2.  The plan minimises sum_c cost_hc(t_c),
 * cost_hc(t) = fl64(fl64(q_hc^2 * delta_c^2) * E_c(t)), delta_c =
 * fl32(fl32(hi - lo) * 1/16), over all plans with sum t_c = B, 0 <= t_c <= 4
 * (dynamic programming over the channels in order, fp64 sums; on equal sums
 * the smaller t of the later channel wins).  Unlike fill-to-cap it skips
 * depths that leave more error than reading less (a channel whose keys sit
 * near its range's midpoint gains nothing from its top bit).
 *   q            device fp32[hq][d];  lo, hi device fp32[hkv][d] (fathom_pack)
 *   hist         device uint32[hkv][d][16] (fathom_code_hist)
 *   budget_bits  HOST int32[hq], each in [0, 4d]
 *   plan         device output uint8[hq][d], sum_c t_c = B.                  */
int32_t fathom_code_hist(const uint32_t *planes, int64_t n, int32_t hkv, int32_t d,
                         int64_t plane_words, uint32_t *hist, void *stream);
int32_t fathom_plan_calibrated(const float *q, int32_t hq, int32_t hkv, int32_t d,
                               const float *lo, const float *hi,
                               const uint32_t *hist, const int32_t *budget_bits,
                               uint8_t *plan, void *stream);
/* The same allocation once per GQA group (as fathom_plan_group does for the
 * walk): the group's weight of channel c is delta_c^2 times the fp64 sum, in
 * head order, of q_hc^2 over its heads; budget_bits is HOST int32[hkv]; every
 * head of the group receives the row.  With one head per group it equals
 * fathom_plan_calibrated.                                                   */
int32_t fathom_plan_calibrated_group(const float *q, int32_t hq, int32_t hkv, int32_t d,
                                     const float *lo, const float *hi,
                                     const uint32_t *hist, const int32_t *budget_bits,
                                     uint8_t *plan, void *stream);

/* Fixed-width baseline plan (the pages' 136-bit scans read r = 32 channels
 * in full): the r channels with the largest |q_c| (ties: lower channel) get
 * t = 4, all others 0.  0 <= r <= d.                                        */
int32_t fathom_plan_fixed(const float *q, int32_t hq, int32_t d, int32_t r,
                          uint8_t *plan, void *stream);

/* ---- scan ----------------------------------------------------------------
 * Explainer, section 核心方法 (read side) and problem statement: each query
 * head reads only the top t_c planes of every channel and scores all n keys.
 * The unread low bits are reconstructed at their midpoint:
 *   s_i = sum_c q_c * (lo_c + (floor(code_ic / 2^(4-t_c)) + 1/2) *
 *                       delta_c * 2^(4-t_c))   [+ meta_scale * meta[g][i]]
 * Per kv head the planes read are the union of its query heads' plans, read
 * once for the whole group.  Accuracy: |s - exact| <= 1e-5 * A_h with
 * A_h = sum_c |q_c| * max(|lo_c|, |hi_c|).
 *
 * planes      device (HBM) or pinned host memory, layout of fathom_pack.
 * lo, hi      device fp32[hkv][d]
 * q           device fp32[hq][d];  plan  device uint8[hq][d] (t in 0..4)
 * meta        NULL, or device/pinned uint8[hkv][n]: an 8-bit per-key side
 *             stream added as meta_scale * meta (fixed-width baseline).
 * logits      device output fp32[hq][ld_logits], ld_logits >= n; only
 *             columns < n are written.                                      */
int32_t fathom_scan(const uint32_t *planes, const float *lo, const float *hi,
                    int64_t n, int32_t hkv, int32_t d, const float *q,
                    const uint8_t *plan, int32_t hq, const uint8_t *meta,
                    float meta_scale, float *logits, int64_t ld_logits,
                    void *stream);

/* ---- top-k ---------------------------------------------------------------
 * Explainer, problem statement: every decode step keeps the top k of the n
 * scored keys.  Ranking: score descending, then index ascending.  With
 * group = G > 1 each output row o ranks the group score
 *   S_i = fp32( ((0 + s[oG][i]) + s[oG+1][i]) + ... ) added in fp64.
 * -0.0 ranks equal to +0.0.  Rows with n < k are padded with idx -1 and
 * score -inf.  Results are identical to a full sort.
 *
 * scores  device fp32[rows][ld], ld >= n;  rows % group == 0
 * idx     device output int32[rows/group][k];  vals  fp32[rows/group][k]
 *         (the ranked scores, in rank order)
 * ws      device workspace, >= fathom_topk_workspace_bytes(rows/group, k).
 * 1 <= k <= FATHOM_MAX_K, 0 <= n < 2^31.                                    */
int32_t fathom_topk(const float *scores, int32_t rows, int64_t n, int64_t ld,
                    int32_t group, int32_t k, int32_t *idx, float *vals,
                    void *ws, int64_t ws_bytes, void *stream);

/* ---- top-k for callers that cannot allocate -------------------------------
 * For callers that cannot call hipMalloc or pass a workspace (code under HIP
 * graph capture, serving loops that forbid allocation): fathom_topk with its
 * workspace taken from a static device array inside the library, of
 * FATHOM_NOALLOC_MAX_ROWS output rows (about 4 MiB per GPU, held from the
 * library's load until the process ends).  Same arguments, ranking, padding
 * and results as fathom_topk, minus ws / ws_bytes; allocates nothing.
 * rows / group > FATHOM_NOALLOC_MAX_ROWS -> FATHOM_ERR_WORKSPACE.  Every
 * call on one GPU uses that GPU's one array (the kernels reset what must
 * start at zero): calls that overlap on one GPU (two streams, or two host
 * threads without ordering) race and must be ordered by the caller.        */
#define FATHOM_NOALLOC_MAX_ROWS 64
int32_t fathom_topk_noalloc(const float *scores, int32_t rows, int64_t n, int64_t ld,
                            int32_t group, int32_t k, int32_t *idx, float *vals,
                            void *stream);

/* ---- many sessions in one launch ----------------------------------------
 * Ragged multi-session decode: every session has its own K cache (planes,
 * lo, hi of n keys), its own queries and plan; one launch scans all sessions
 * (work spread over (session, kv head, key tile)), and one set of launches
 * selects all sessions' top-k.  The descriptor array is HOST memory, read
 * during the call only.  Fields not used by a call may be NULL.            */
typedef struct {
  const uint32_t *planes; /* device or pinned host, fathom_pack layout      */
  const float *lo, *hi;   /* device fp32[hkv][d]                            */
  int64_t n;              /* keys in this session (>= 0)                    */
  const float *q;         /* device fp32[hq][d]                             */
  const uint8_t *plan;    /* device uint8[hq][d]                            */
  const uint8_t *meta;    /* NULL or uint8[hkv][n]                          */
  float meta_scale;
  float *logits;          /* device fp32[hq][ld_logits]                     */
  int64_t ld_logits;
  int32_t *idx;           /* device int32[hq/group][k] (top-k output)       */
  float *vals;            /* device fp32[hq/group][k]                       */
  int64_t plane_words;    /* row length W of planes in words: 0 means       */
                          /* fathom_plane_words(n); a larger capacity (a    */
                          /* multiple of 64, <= 2^26) lets a session grow by */
                          /* fathom_append without moving its planes        */
} fathom_session;

int32_t fathom_scan_batched(const fathom_session *sessions, int32_t n_sessions,
                            int32_t hkv, int32_t d, int32_t hq, void *stream);
int32_t fathom_topk_batched(const fathom_session *sessions, int32_t n_sessions,
                            int32_t hq, int32_t group, int32_t k, void *ws,
                            int64_t ws_bytes, void *stream);

/* ---- scan + top-k in one call --------------------------------------------
 * Explainer, problem statement (every decode step scores the n keys and keeps
 * the top k) with the scan of section 核心方法 (read side): idx and vals are
 * those of fathom_scan followed by fathom_topk on the same inputs (same
 * scores, ranking, tie order and padding), but the logits of all keys are
 * not written unless needed.  With planes in device memory, n <= 2^25 and
 * group 1 or hq/hkv (<= 4), the call scores a sample of 32 key tiles (2048
 * keys each, the middle tiles of 32 equal stretches of the row; all tiles of
 * shorter rows), sets a per-row threshold from a quarter of their keys,
 * scans again keeping only the (score, index) pairs at or above the
 * threshold, and ranks those; a row whose candidate count falls outside
 * [k, 8192] is recomputed from full logits in the workspace (by the last
 * block of its kv head's recompute scan, whose launch also holds the
 * ranking blocks of the other rows).  Otherwise (pinned host planes, other
 * groups, longer sessions) the full logits go to the workspace and are
 * ranked there.
 *
 * Arguments as for fathom_scan and fathom_topk (group over the hq rows);
 * idx, vals  device outputs int32/fp32[hq/group][k].
 * ws         device workspace of fathom_scan_topk_workspace_bytes bytes.
 * Enqueues four kernel launches (sample scan, threshold, candidate scan,
 * ranking + recompute scan; the scans once more per further 4 query heads
 * of a kv head or 16 sessions, and the ranking as a launch of its own when
 * a session has no keys); nothing synchronises.                            */
int64_t fathom_scan_topk_workspace_bytes(const int64_t *n_host, int32_t n_sessions,
                                         int32_t hkv, int32_t hq, int32_t group,
                                         int32_t k);
int32_t fathom_scan_topk(const uint32_t *planes, const float *lo,
                         const float *hi, int64_t n, int32_t hkv, int32_t d,
                         const float *q, const uint8_t *plan, int32_t hq,
                         const uint8_t *meta, float meta_scale, int32_t group,
                         int32_t k, int32_t *idx, float *vals, void *ws,
                         int64_t ws_bytes, void *stream);
/* Many sessions: descriptors as for fathom_scan_batched (logits and
 * ld_logits ignored; idx, vals required).  n_host of the workspace query
 * lists the sessions' n in order.                                           */
int32_t fathom_scan_topk_batched(const fathom_session *sessions,
                                 int32_t n_sessions, int32_t hkv, int32_t d,
                                 int32_t hq, int32_t group, int32_t k, void *ws,
                                 int64_t ws_bytes, void *stream);

/* ---- the 68-bit fixed-width baseline --------------------------------------
 * Explainer, key-experiments section (关键实验与数据): Fathom is compared with
 * the fixed r = 16 scan at 68 bits per key, and with fixed 136-bit scans at
 * r = 32.  Both are 4.25 r bits: 4 bits of each of r channels plus r/4 bits
 * of per-key metadata (a reading; the pages do not lay the metadata out).
 * The 136-bit form's 8-bit stream is fathom_scan's `meta`; these calls carry
 * the r = 16 form's 4-bit stream:
 *   meta4  device or pinned-host uint8[hkv][ceil(n/2)], two keys per byte:
 *          key i of kv head g is the low nibble of meta4[g][i/2] when i is
 *          even, the high nibble when i is odd; it adds meta_scale * value.
 * Otherwise as fathom_scan and fathom_scan_topk (typically with a plan from
 * fathom_plan_fixed with r = 16).  meta4 may be NULL only when n == 0.     */
int32_t fathom_scan_meta4(const uint32_t *planes, const float *lo, const float *hi,
                          int64_t n, int32_t hkv, int32_t d, const float *q,
                          const uint8_t *plan, int32_t hq, const uint8_t *meta4,
                          float meta_scale, float *logits, int64_t ld_logits,
                          void *stream);
int32_t fathom_scan_topk_meta4(const uint32_t *planes, const float *lo, const float *hi,
                               int64_t n, int32_t hkv, int32_t d, const float *q,
                               const uint8_t *plan, int32_t hq, const uint8_t *meta4,
                               float meta_scale, int32_t group, int32_t k, int32_t *idx,
                               float *vals, void *ws, int64_t ws_bytes, void *stream);

/* ---- append (decode-time growth) -------------------------------------------
 * Deployment warnings, item 3: the planes are the stored 4-bit K itself, so
 * nothing else is rebuilt when K changes; a decode step adds its new keys to
 * the stored K.  Here the m new keys become tokens n_old .. n_old+m-1 of a
 * packed layer, quantised with the layer's stored range (no re-quantisation
 * of earlier keys): code = floor((x - lo) / delta) with fp32 subtract and
 * divide, delta = (hi - lo) * 1/16, clamped to 0..15; delta == 0 gives 0.
 * sigma2 is left as stored.  Only those tokens' bits change.
 *
 * keys        device rows of `dtype`: element (new token j, kv head h,
 *             channel c) at keys[j*stride_tok + h*stride_head + c]
 * planes      device or pinned-host uint32[hkv][d][4][plane_words], rows of
 *             plane_words >= fathom_plane_words(n_old + m) words, a multiple
 *             of 64 (a capacity; scans of the grown layer pass it in
 *             fathom_session.plane_words)
 * lo, hi      device fp32[hkv][d] as stored by fathom_pack
 * clamped     NULL, or a device uint32 to which the number of values outside
 *             [lo, hi] is added (the caller may re-pack when it grows)
 * Enqueues 1 kernel (none when m == 0).  Calls that write the same plane
 * words (appends to one layer) must be ordered on one stream.              */
int32_t fathom_append(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                      int32_t d, int64_t stride_tok, int64_t stride_head,
                      int64_t n_old, uint32_t *planes, int64_t plane_words,
                      const float *lo, const float *hi, uint32_t *clamped,
                      void *stream);

/* ---- per-block ranges ------------------------------------------------------
 * Explainer, deployment warnings item 3 (the bit planes ARE the stored 4-bit
 * K: changing its quantisation must not force anything else to be rebuilt)
 * and problem statement (long sessions that grow by one key per decode
 * step).  The pages keep one range per channel; a session whose key ranges
 * drift would then either clamp its later keys or re-quantise every stored
 * code.  Reading taken here: the range of a channel is kept per block of
 * FATHOM_RANGE_BLOCK = 2048 consecutive keys (one 64-word block of every
 * plane row), so later blocks get ranges of their own and no stored code is
 * ever re-quantised.  Planes keep the fathom_pack layout.
 *
 * lo, hi       device fp32[hkv][range_stride][d]: block b of channel c of kv
 *              head h at [(h*range_stride + b)*d + c] (one block's d ranges
 *              are contiguous); range_stride is a capacity,
 *              fathom_range_blocks(n) <= range_stride <= 2^20.
 *
 * fathom_pack_blocked: each block's range is the min and max of its own keys
 * (-0 stored as +0); its keys are coded with it exactly as fathom_pack codes
 * a layer (delta_b = (hi_b - lo_b) * 1/16, code = min(15, floor((x - lo_b) /
 * delta_b)), delta_b == 0 gives 0).  sigma2 (device fp32[hkv][d]) is the
 * pooled within-block variance of the dequantised values:
 *   sigma2 = fp32( sum over blocks in order of fp64(var_b * (n_b / n)) ),
 *   var_b  = fp64((n_b*S2_b - S1_b^2) / n_b^2) * delta_b^2   (fp64 steps),
 * with n_b the block's keys and S1_b, S2_b its code sums; a layer of one
 * block gets fathom_pack's sigma2.  ws: fathom_pack_blocked_workspace_bytes.
 * Other arguments as fathom_pack.  Outputs are bit-identical to the CPU
 * definition.  Enqueues 3 kernels.
 *
 * fathom_append_blocked: as fathom_append, except that a block which holds no
 * key before the call first takes the range of the block before it, widened
 * to cover the keys the call puts in it (block 0: those keys' own min and
 * max); a block that already holds keys keeps its range, and keys outside it
 * are clamped and counted in `clamped`.  lo and hi are read and written.
 * Enqueues 1 to 3 kernels (none when m == 0).
 *
 * fathom_scan_blocked: fathom_scan with key i reading lo_b, delta_b of its
 * block b = i / 2048 in the reconstruction formula (no side stream);
 * plane_words as fathom_session.plane_words (0: fathom_plane_words(n)).
 * Accuracy |s - exact| <= 1e-5 * A_h, A_h = sum_c |q_c| * max over blocks of
 * max(|lo_cb|, |hi_cb|).
 *
 * fathom_scan_topk_blocked: fathom_scan_topk over the per-block scan (same
 * ranking, ties and padding; workspace from fathom_scan_topk_workspace_bytes).
 */
#define FATHOM_RANGE_BLOCK 2048
int64_t fathom_range_blocks(int64_t n);
int64_t fathom_pack_blocked_workspace_bytes(int64_t n, int32_t hkv, int32_t d);
int32_t fathom_pack_blocked(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                            int32_t d, int64_t stride_tok, int64_t stride_head,
                            uint32_t *planes, float *lo, float *hi, int64_t range_stride,
                            float *sigma2, void *ws, int64_t ws_bytes, void *stream);
int32_t fathom_append_blocked(const void *keys, int32_t dtype, int64_t m, int32_t hkv,
                              int32_t d, int64_t stride_tok, int64_t stride_head,
                              int64_t n_old, uint32_t *planes, int64_t plane_words,
                              float *lo, float *hi, int64_t range_stride,
                              uint32_t *clamped, void *stream);
int32_t fathom_scan_blocked(const uint32_t *planes, const float *lo, const float *hi,
                            int64_t range_stride, int64_t n, int32_t hkv, int32_t d,
                            const float *q, const uint8_t *plan, int32_t hq,
                            int64_t plane_words, float *logits, int64_t ld_logits,
                            void *stream);
int32_t fathom_scan_topk_blocked(const uint32_t *planes, const float *lo, const float *hi,
                                 int64_t range_stride, int64_t n, int32_t hkv, int32_t d,
                                 const float *q, const uint8_t *plan, int32_t hq,
                                 int64_t plane_words, int32_t group, int32_t k,
                                 int32_t *idx, float *vals, void *ws, int64_t ws_bytes,
                                 void *stream);

/* ---- sparse attention over the selected keys -------------------------------
 * Explainer, problem statement: each generated token attends over the top k
 * of its n keys; the future-work list keeps V dense.  The pages do not lay
 * this step out.  Here the selected keys' full-precision K and V rows are
 * gathered (token-major, in HBM or pinned host memory) and, per query head h
 * with kv head g = h / (hq / hkv), over the entries of its index row:
 *   s_i = scale * sum_c q_hc K_igc   (fp32 products and sums: runs of 8
 *                                     (fp16) or 4 (fp32) channels in order,
 *                                     their sums by a butterfly)
 *   m = max s_i, p_i = exp(s_i - m), out_h = sum_i p_i V_ig / sum_i p_i,
 *   lse_h = m + log(sum_i p_i)       (natural log)
 * in fp32 (partials (m, sum p, sum p V) over at most 64 entries each,
 * merged by maxima).
 *
 * q        device fp32[hq][d]
 * k_cache, v_cache  device or pinned-host rows of `dtype` (FATHOM_F16 or
 *          FATHOM_F32); element (token i, kv head g, channel c) at
 *          [i*stride_tok + g*stride_head + c].  Both 16-byte aligned, strides
 *          multiples of 16 bytes (else FATHOM_ERR_UNSUPPORTED).  May be NULL
 *          when n == 0.
 * idx      device int32[hq/group][k]: row o serves query heads o*group ..
 *          o*group+group-1 (group 1, 2, 4 or 8, dividing hq/hkv); e.g. the
 *          idx of fathom_topk / fathom_scan_topk with the same group.
 *          Entries < 0 (the padding of short rows) or >= n are skipped
 *          without any memory access; an entry listed twice counts twice.
 *          May be NULL when k == 0.
 * scale    finite softmax scale (1/sqrt(d) for standard attention).
 * out      device output fp32[hq][d]; lse device output fp32[hq].  A head
 *          with no valid entry gets out = 0 and lse = -inf.
 * ws       device workspace of fathom_attention_workspace_bytes(hq, k)
 *          bytes (may be NULL when k == 0).
 * Enqueues 2 kernels; 0 <= k <= FATHOM_MAX_ATTN_K.                         */
int64_t fathom_attention_workspace_bytes(int32_t hq, int32_t k);
int32_t fathom_sparse_attention(const float *q, int32_t hq, int32_t hkv, int32_t d,
                                const void *k_cache, const void *v_cache,
                                int32_t dtype, int64_t n, int64_t stride_tok,
                                int64_t stride_head, const int32_t *idx,
                                int32_t group, int32_t k, float scale, float *out,
                                float *lse, void *ws, int64_t ws_bytes,
                                void *stream);

/* ---- observability -------------------------------------------------------
 * The plane reads themselves, for bit-exact checks: out[h][i][c] =
 * floor(code_ic / 2^(4-t_hc)) (0 where t = 0).  out device uint8[hq][n][d]. */
int32_t fathom_read_prefixes(const uint32_t *planes, int64_t n, int32_t hkv,
                             int32_t d, const uint8_t *plan, int32_t hq,
                             uint8_t *out, void *stream);

/* Explainer, section 对工程落地的启发 (engineering notes): the bits each
 * channel reads should be observable per query.  HOST-only: from a host copy
 * of a plan, hist[t] = number of (head, channel) pairs read at depth t
 * (t = 0..4), union_bits[g] = sum_c max_{h in group g} t_hc = plane bits per
 * key that group g's scan reads.  union_bits may be NULL.                   */
int32_t fathom_plan_stats(const uint8_t *plan_host, int32_t hq, int32_t d,
                          int32_t group, uint32_t *hist,
                          uint32_t *union_bits);

/* Streaming-read probe used as the roofline denominator: reads `bytes` from
 * `src` (device or pinned host, 16-byte aligned, bytes % 16 == 0) with every
 * CU and writes one checksum word to device `out` (uint32[1]).  `blocks`
 * = 0 picks a default grid.                                                 */
int32_t fathom_probe_read(const void *src, int64_t bytes, uint32_t *out,
                          int32_t blocks, void *stream);

/* Scan-traffic probe, the measured ceiling for an HBM-resident logits scan's
 * own access pattern: it moves the bytes that scan moves with none of its
 * arithmetic.  Device planes [hkv][128][4][n/32] (16-byte aligned), device
 * depth uint8[hkv][128] (plane slots read per channel, clamped to 0..4; for
 * a scan, the largest t_hc of the kv head's query heads).  Per 2048-key tile
 * of each kv head it reads, with 16-byte lanes, the tile's 256 bytes of
 * every plane row below the channel's depth, and writes rows_out (0..16)
 * device fp32 rows of the tile: out row g*rows_out + r, row stride ld >= n
 * (ld % 4 == 0; out 16-byte aligned; unused when rows_out == 0).  The values
 * written carry no meaning; one checksum word goes to device sink
 * (uint32[1]).  n > 0 and a multiple of 2048, hkv 1..64.  One kernel.       */
int32_t fathom_probe_scan_traffic(const uint32_t *planes, int64_t n, int32_t hkv,
                                  const uint8_t *depth, int32_t rows_out, float *out,
                                  int64_t ld, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FATHOM_H */
