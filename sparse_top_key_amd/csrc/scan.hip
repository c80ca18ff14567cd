// Variable-depth plane scan (explainer, section 核心方法, read side): every
// query head reads only the top t_c planes of each channel and scores all n
// keys; the unread low bits sit at their midpoint.
//
// Arithmetic.  With delta_c = (hi_c - lo_c)/16 and m = the value of the top
// t planes placed at their own bit positions (code with its low 4-t bits
// cleared),
//     s_i = C_h + sum_c gamma_hc * m_ic,
//     gamma_hc = q_hc * delta_c            (0 when t_hc = 0),
//     C_h = sum_c q_hc * (lo_c + delta_c * 2^(3 - t_hc))   (fp64, rounded once).
//
// Slots (both kernels): the distinct (channel, depth) pairs the query heads
// of one kv head read.  A slot of depth u loads the top u planes of its
// channel, so the union of the heads' reads comes from memory once; each head
// weighs exactly the slots at its own depths.  Slots are ordered by the set
// of heads that use them, then by channel, and handled 8 at a time: 32 plane
// rows (8 slots x 4 planes, unread planes = 0), bit-transposed so that every
// key gets one word of 8 nibble codes.
//
// Two kernels (the pages give no kernel design; both are MI355X-first):
//  * scan_mfma_kernel, planes in HBM: the contraction over slots runs on the
//    matrix cores with exact int8 limbs of gamma (see its comment).
//  * scan_kernel, planes in pinned host memory (and sessions above 2^25
//    keys): the link is the bound, so the fp32 FMA form is enough.  A block
//    takes one (session, kv head) and a run of 8192-key tiles; its 4 waves
//    take 2048 keys each: lane w owns plane word w (keys 32w..32w+31), so
//    every plane load is one coalesced 256-byte wave access.  Nibbles become
//    fp32 through byte conversions, then one FMA per (head, slot, key), with
//    the weights in scalar registers; the next 8 slots' words are loaded
//    while the current ones are computed.  The per-key sum has one fp32 term
//    per channel read, so its rounding error is bounded by
//    (terms + 1) * 2^-24 * sum|terms|, well inside 1e-5 * A_h.
#include <climits>
#include <type_traits>

#include "fathom_internal.h"
#include "select.h"

namespace fathom {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMinSetupThreads = 256;             // smallest block building a slot table
constexpr int kMaxSlots = kD * kPlanes;           // (channel, depth) pairs
constexpr int kMaxGroups = kMaxSlots / 8;

struct ScanSess {
  const uint32_t *planes;
  const float *lo, *hi, *q;
  const uint8_t *plan, *meta;
  int32_t meta_bits;       // side stream: 8 (a byte per key) or 4 (two keys per byte)
  float *logits;
  int64_t n, W, ld;
  float meta_scale;
  int32_t block_begin;     // first block of this session in the grid
  int32_t tiles_per_block;
  int32_t blocks_per_head;
  int32_t vec_out;         // float4 logits stores are aligned
  // tiles this launch visits (all, or the sampled ones) and real tiles
  int32_t nvtiles, ntiles;
  // fused scan + top-k
  uint16_t *sample;
  const uint32_t *thr;
  uint64_t *cand;
  uint32_t *seg_cnt;
  uint32_t *ovf_cnt;
  uint64_t *ovf;
  // recompute scan of a fused call (null otherwise): blocks finished per
  // (kv head, head chunk), the outputs, and the records of recomputed rows
  // and kv heads that the final blocks set
  uint32_t *redo_done;
  uint32_t *redo;
  uint32_t *row_flag;
  int32_t *out_idx;
  float *out_vals;
  int32_t seg_cap;         // candidate words per (row, block) segment
  int32_t nseg;            // recompute scan: the candidate scan's segments per row
  uint8_t *table;          // slot records of the session, or null
  int32_t table_mode;      // ScanTable
  int64_t rs;              // 0: lo, hi [hkv][d]; > 0: per 2048-key block, [hkv][rs][d]
};

struct ScanArgs {
  ScanSess s[kSessPerLaunch];
  int32_t n_sess, hkv, group, head0;
  int32_t out_k, out_group;  // recompute scan: outputs per row; query heads per row
  // recompute scan: blocks 0 .. n_final-1 are the fused final's, one per
  // output row (final_rows per session) ahead of the scan blocks
  int32_t n_final, final_rows;
};
static_assert(sizeof(ScanArgs) <= 4096, "kernel arguments");

// The kernels read their descriptors in place from the kernel-argument
// segment (address space 4): indexing them by session then needs no copy.
typedef __attribute__((address_space(4))) const ScanArgs KScanArgs;
typedef __attribute__((address_space(4))) const ScanSess KScanSess;

// ---- 32x32 bit transpose ----------------------------------------------------
// On entry x[r] bit k = element (r, k); on exit x[k] bit r = element (r, k).
// Stage S swaps the off-diagonal SxS blocks of every 2Sx2S block.
template <int N, int S, uint32_t M>
__device__ __forceinline__ void transpose_stage(uint32_t (&x)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) {
    if ((r & S) == 0) {
      const uint32_t a = x[r], b = x[r + S];
      x[r] = (a & M) | ((b << S) & ~M);
      x[r + S] = ((a >> S) & M) | (b & ~M);
    }
  }
}

__device__ __forceinline__ void transpose32(uint32_t (&x)[32]) {
  transpose_stage<32, 16, 0x0000FFFFu>(x);
  transpose_stage<32, 8, 0x00FF00FFu>(x);
  transpose_stage<32, 4, 0x0F0F0F0Fu>(x);
  transpose_stage<32, 2, 0x33333333u>(x);
  transpose_stage<32, 1, 0x55555555u>(x);
}

// The same transpose; the two byte-granular stages (16 and 8) use one byte
// permute per output word.
__device__ __forceinline__ void transpose32_perm(uint32_t (&x)[32]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t a = x[r], b = x[r + 16];
    x[r] = __builtin_amdgcn_perm(b, a, 0x05040100u);       // a.lo16 | b.lo16 << 16
    x[r + 16] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi16 | b.hi16 << 16
  }
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if ((r & 8) == 0) {
      const uint32_t a = x[r], b = x[r + 8];
      x[r] = __builtin_amdgcn_perm(b, a, 0x06020400u);      // bytes a0 b0 a2 b2
      x[r + 8] = __builtin_amdgcn_perm(b, a, 0x07030501u);  // bytes a1 b1 a3 b3
    }
  }
  transpose_stage<32, 4, 0x0F0F0F0Fu>(x);
  transpose_stage<32, 2, 0x33333333u>(x);
  transpose_stage<32, 1, 0x55555555u>(x);
}

__device__ __forceinline__ int uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ float uniform_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// The 8 nibbles of a transposed word as fp32 values: two masks split the
// nibbles into the low halves of bytes, then one byte conversion each.
__device__ __forceinline__ void nibbles_to_f32(uint32_t y, float (&f)[8]) {
  const uint32_t e = y & 0x0F0F0F0Fu;         // slots 0, 2, 4, 6
  const uint32_t o = (y >> 4) & 0x0F0F0F0Fu;  // slots 1, 3, 5, 7
  asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f[0]) : "v"(e));
  asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f[1]) : "v"(o));
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f[2]) : "v"(e));
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f[3]) : "v"(o));
  asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f[4]) : "v"(e));
  asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f[5]) : "v"(o));
  asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f[6]) : "v"(e));
  asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f[7]) : "v"(o));
}

// Rows 4j+p of x receive bit p of slot (grp*8 + j)'s code: plane slot 3-p of
// its channel, loaded only when it lies in the slot's plane range.  Loads are
// buffer loads: a wave-uniform resource per channel (its 4 plane rows), a
// wave-uniform row + block offset, and the lane's 32-bit byte offset `voff`.
// The resource's size also bounds every access.
constexpr int32_t kRsrcWord3 = 0x00020000;

template <int AUX>
__device__ __forceinline__ void load_group(const uint32_t *__restrict__ gplanes, int64_t W,
                                           int32_t wbase, uint32_t voff,
                                           const int16_t *slot_desc, int grp,
                                           uint32_t (&x)[32]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int desc = uniform(slot_desc[grp * 8 + j]);
    const int c = (desc >> 3) & (kD - 1), dep = desc & 7, top = desc >> 10;
    const uint32_t *pc = gplanes + (int64_t)c * kPlanes * W;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(pc), (short)0, (int32_t)(W * kPlanes * 4), kRsrcWord3);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t v = 0;
      if (3 - p < dep && 3 - p >= top)
        v = __builtin_amdgcn_raw_buffer_load_b32(
            rsrc, (int32_t)voff, (int32_t)(((3 - p) * W + wbase) * 4), AUX);
      x[4 * j + p] = v;
    }
  }
}

// ---- slot table (per block: one session, one kv head, GH query heads) ------
// Slots are the distinct (channel, depth) pairs the GH heads read.  With
// u_1 < u_2 < ... the distinct depths of channel c among the heads, slot
// (c, u_k) stands for the plane slots u_{k-1} .. u_k - 1 of the channel
// (u_0 = 0), placed at their own bit positions, so every plane is loaded once
// per channel; a head reading c to depth t uses the slots with u_k <= t, each
// with weight gamma = q_hc * delta_c, and their values add up to its top t
// planes.  Slots are ordered by the set of heads using them (larger sets
// first), then channel, then depth.
template <int GH>
struct SlotTable {
  int16_t desc[kMaxSlots];       // (u_{k-1} << 10) | (channel << 3) | u_k; 0 = padding
  float gam[kMaxSlots][GH];      // gamma per slot and head (0: head does not use it)
  uint8_t gmask[kMaxGroups];     // heads using any slot of an 8-slot group
  float C[GH];                   // C_h = sum_c q_hc (lo_c + delta_c 2^(3 - t_hc))
  uint32_t gmax[GH];             // bits of max |gamma| per head (non-negative floats)
  int nslots;
};

// Set-up-only storage; the matrix-core kernel overlays it on its code table.
constexpr int kCandWaves = kD * 4 / 64;  // (channel, depth) candidates in waves of 64
template <int GH>
struct SlotScratch {
  float q[GH][kD];
  float delta[kD];
  uint8_t t[GH][kD];
  double cpart[2][GH];           // C_h halves (channels 0..63, 64..127)
  int wcnt[kCandWaves][16];      // slots of each membership class per candidate wave
  int wpre[kCandWaves][16];      // ... in the earlier candidate waves
  int cbase[16];                 // first rank of each class
};

// Rank of a membership set (bit j: head j uses the slot) in the slot order:
// more heads first, then by the set's value (15 marks "no slot").
__device__ __forceinline__ int memb_class(int memb) {
  // nibble m = class of set m: 15; 7 11 13 14; 3 5 6 9 10 12; 1 2 4 8; none
  constexpr uint64_t kClass = 0x043A298E176D5CBFull;
  return (int)((kClass >> (4 * memb)) & 15u);
}

// The slot table of one (session, kv head) and the GH query heads from
// head_base.  Every step is parallel: per-channel terms in registers, C_h by
// wave shuffles in a fixed fp64 order, slot ranks by counting ballots per
// membership class, the per-head max |gamma| by LDS atomics.  Per-block
// ranges (S.rs > 0): the table is built with delta = 1 and lo = 0, so that
// gam holds q_hc for the heads using the slot (each scan block then forms
// its own gamma and C_h per 2048-key block).
template <int GH>
__device__ void build_slot_table(SlotTable<GH> &T, SlotScratch<GH> &X, KScanSess &S, int g,
                                 int head_base) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (tid < kD) {
    const int c = tid;
    const bool unit = S.rs > 0;
    const float lo = unit ? 0.0f : S.lo[g * kD + c];
    const float hi = unit ? 16.0f : S.hi[g * kD + c];
    int t[GH];
    float q[GH];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      t[j] = S.plan[(int64_t)(head_base + j) * kD + c];
      q[j] = S.q[(int64_t)(head_base + j) * kD + c];
    }
    const float delta = __fmul_rn(__fsub_rn(hi, lo), 0.0625f);
    X.delta[c] = delta;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      X.t[j][c] = (uint8_t)t[j];
      X.q[j][c] = q[j];
      // C_h term q * (lo + delta * 2^(3-t)) in fp64 (exact operands), summed
      // over the 64 channels of the wave by a butterfly
      const double mid = (double)lo + (double)delta * (double)(1 << (4 - t[j])) * 0.5;
      double v = (double)q[j] * mid;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v = __dadd_rn(v, __shfl_xor(v, off));
      if (lane == 0) X.cpart[tid >> 6][j] = v;
    }
  }
  if (tid < GH) T.gmax[tid] = 0u;
  __syncthreads();
  if (tid < GH) T.C[tid] = (float)__dadd_rn(X.cpart[0][tid], X.cpart[1][tid]);
  // ---- candidates (channel, depth) = e: membership class, counts per wave
  constexpr int kIters = kD * 4 / kMinSetupThreads;
  int memb_e[kIters], cls_e[kIters], pre_e[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int e = tid + it * blockDim.x;
    memb_e[it] = 0;
    cls_e[it] = 15;
    pre_e[it] = 0;
    if (e >= kD * 4) continue;  // blocks of more than kD*4 threads
    const int c = e >> 2, dep = (e & 3) + 1;
    int memb = 0;
    bool exact = false;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      memb |= (X.t[j][c] >= dep) << j;
      exact |= X.t[j][c] == dep;
    }
    const int k = exact ? memb_class(memb) : 15;
    const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int kk = 0; kk < 15; ++kk) {
      const uint64_t m = __ballot(k == kk);
      if (k == kk) pre_e[it] = __popcll(m & lt);
      if (lane == 0) X.wcnt[e >> 6][kk] = __popcll(m);
    }
    memb_e[it] = memb;
    cls_e[it] = k;
  }
  __syncthreads();
  // class bases and per-wave prefixes (16 lanes of wave 0)
  if (tid < 16) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kCandWaves; ++w) {
      const int cnt = tid < 15 ? X.wcnt[w][tid] : 0;
      X.wpre[w][tid] = run;
      run += cnt;
    }
    // exclusive scan of the class totals over the 16 lanes
    int incl = run;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(incl, off, 16);
      if (tid >= off) incl += o;
    }
    X.cbase[tid] = incl - run;
    if (tid == 15) T.nslots = incl;
  }
  __syncthreads();
  const int nslots = T.nslots;
  const int ngroups = (nslots + 7) >> 3;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int e = tid + it * blockDim.x;
    const int k = cls_e[it];
    if (e >= kD * 4 || k == 15) continue;
    const int c = e >> 2, dep = (e & 3) + 1;
    const int rank = X.cbase[k] + X.wpre[e >> 6][k] + pre_e[it];
    int top = 0;  // the next smaller depth read in this channel
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const int tj = X.t[j][c];
      if (tj < dep && tj > top) top = tj;
    }
    T.desc[rank] = (int16_t)((top << 10) | (c << 3) | dep);
    const float delta = X.delta[c];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const float gm = ((memb_e[it] >> j) & 1) ? __fmul_rn(X.q[j][c], delta) : 0.0f;
      T.gam[rank][j] = gm;
      atomicMax(&T.gmax[j], __float_as_uint(fabsf(gm)));
    }
  }
  for (int e = nslots + tid; e < ngroups * 8; e += blockDim.x) {
    T.desc[e] = 0;
#pragma unroll
    for (int j = 0; j < GH; ++j) T.gam[e][j] = 0.0f;
  }
  __syncthreads();
  for (int gi = tid; gi < ngroups; gi += blockDim.x) {
    int m = 0;
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int h = 0; h < GH; ++h) m |= (T.gam[gi * 8 + j][h] != 0.0f) << h;
    T.gmask[gi] = (uint8_t)m;
  }
  __syncthreads();
}

// Block -> (session, kv head, first tile); tiles are taken with a stride of
// the number of blocks per head so that blocks running together stream
// neighbouring addresses.
struct BlockWork {
  KScanSess *S;
  int g, tile0, tile_step, head_base;
  int rec;  // slot record of (kv head, head chunk) in the session's tables
};

__device__ __forceinline__ BlockWork block_work(const ScanArgs &) {
  // the descriptors are read in place from the kernel-argument segment (the
  // kernels' only argument), so indexing them does not copy them to scratch
  KScanArgs &a = *(KScanArgs *)__builtin_amdgcn_kernarg_segment_ptr();
  int si = 0;
  for (int j = 1; j < a.n_sess; ++j)
    if ((int)blockIdx.x >= a.s[j].block_begin) si = j;
  BlockWork w;
  w.S = &a.s[si];
  const int local = blockIdx.x - w.S->block_begin;
  w.g = local % a.hkv;
  w.tile0 = local / a.hkv;
  w.tile_step = w.S->blocks_per_head;
  w.head_base = w.g * a.group + a.head0;
  w.rec = w.g * ((a.group + kMaxGH - 1) / kMaxGH) + a.head0 / kMaxGH;
  return w;
}

// Per-block ranges (BLK): a wave's 2048 keys are one range block b, and the
// wave forms that block's weights gamma = q_hc * delta_cb for every slot and
// C_h,b (the same fp64 butterfly as the slot table) before scanning it.
template <int GH>
struct BlockWeights {
  float gam[kScanThreads / 64][kMaxSlots][GH];
  float delta[kScanThreads / 64][kD];
};

template <int GH>
__device__ __forceinline__ void block_weights(BlockWeights<GH> &Wt, const SlotTable<GH> &T,
                                              const SlotScratch<GH> &X, KScanSess &S, int g,
                                              int64_t b, int wave, int lane, float (&C)[GH]) {
  const int64_t r0 = ((int64_t)g * S.rs + b) * kD;  // block b's row of the kv head's ranges
  const float l0 = S.lo[r0 + lane], l1 = S.lo[r0 + lane + 64];
  const float d0 = __fmul_rn(__fsub_rn(S.hi[r0 + lane], l0), 0.0625f);
  const float d1 = __fmul_rn(__fsub_rn(S.hi[r0 + lane + 64], l1), 0.0625f);
  Wt.delta[wave][lane] = d0;
  Wt.delta[wave][lane + 64] = d1;
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    const int t0 = X.t[j][lane], t1 = X.t[j][lane + 64];
    double v0 = (double)X.q[j][lane] *
                ((double)l0 + (double)d0 * (double)(1 << (4 - t0)) * 0.5);
    double v1 = (double)X.q[j][lane + 64] *
                ((double)l1 + (double)d1 * (double)(1 << (4 - t1)) * 0.5);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      v0 = __dadd_rn(v0, __shfl_xor(v0, off));
      v1 = __dadd_rn(v1, __shfl_xor(v1, off));
    }
    C[j] = (float)__dadd_rn(v0, v1);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's deltas are stored
  const int nslots8 = ((T.nslots + 7) >> 3) * 8;
  for (int e = lane; e < nslots8; e += 64) {
    const float dl = Wt.delta[wave][(T.desc[e] >> 3) & (kD - 1)];
#pragma unroll
    for (int j = 0; j < GH; ++j) Wt.gam[wave][e][j] = __fmul_rn(T.gam[e][j], dl);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's weights are stored
}

template <int GH, int AUX, bool BLK>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  const BlockWork bw = block_work(a);
  KScanSess &S = *bw.S;
  const int g = bw.g, tile0 = bw.tile0, tile_step = bw.tile_step, head_base = bw.head_base;
  const int64_t n = S.n;
  __shared__ SlotTable<GH> T;
  __shared__ SlotScratch<GH> X;
  __shared__ typename std::conditional<BLK, BlockWeights<GH>, char>::type Wt;
  build_slot_table<GH>(T, X, S, g, head_base);
  const int tid = threadIdx.x;
  const int ngroups = (T.nslots + 7) >> 3;
  const int16_t *s_desc = T.desc;

  // ---- main loop ------------------------------------------------------------
  // lane = one plane word (32 keys), a wave covers 64 words, and every wave
  // load is one 256-byte access
  constexpr int KPL = 32;
  constexpr int kWaveK = 64 * 32;
  constexpr int kTileK = kWaveK * (kScanThreads / 64);
  const int wave = tid >> 6, lane = tid & 63;
  const uint32_t *gplanes = S.planes + (int64_t)g * kD * kPlanes * S.W;
  float C[GH];
#pragma unroll
  for (int j = 0; j < GH; ++j) C[j] = T.C[j];

  for (int tt = 0; tt < S.tiles_per_block; ++tt) {
    const int64_t wkey0 =
        (int64_t)(tile0 + tt * tile_step) * kTileK + (int64_t)wave * kWaveK;
    if (wkey0 >= n) break;
    const int64_t word = wkey0 / 32 + lane;
    const int32_t wbase = (int32_t)(wkey0 / 32);
    const uint32_t voff = (uint32_t)lane * 4u;  // byte offset
    if constexpr (BLK) block_weights<GH>(Wt, T, X, S, g, wkey0 / kBlockKeys, wave, lane, C);

    float acc[GH][KPL];
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
      for (int k = 0; k < KPL; ++k) acc[j][k] = C[j];

    uint32_t xn[32];
    if (ngroups > 0) load_group<AUX>(gplanes, S.W, wbase, voff, s_desc, 0, xn);
    for (int grp = 0; grp < ngroups; ++grp) {
      uint32_t y[KPL];
#pragma unroll
      for (int r = 0; r < 32; ++r) y[r] = xn[r];
      if (grp + 1 < ngroups) load_group<AUX>(gplanes, S.W, wbase, voff, s_desc, grp + 1, xn);
      transpose32(y);
      const int gm = uniform(T.gmask[grp]);
      // the group's weights, wave-uniform: held in scalar registers
      float gv[GH][8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          if constexpr (BLK)
            gv[h][j] = uniform_f(Wt.gam[wave][grp * 8 + j][h]);
          else
            gv[h][j] = uniform_f(T.gam[grp * 8 + j][h]);
        }
      if (gm == (1 << GH) - 1) {
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          float f[8];
          nibbles_to_f32(y[k], f);
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            float sacc = acc[h][k];
#pragma unroll
            for (int j = 0; j < 8; ++j) sacc = __fmaf_rn(gv[h][j], f[j], sacc);
            acc[h][k] = sacc;
          }
          // keep one key's conversions live at a time (register budget)
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          float f[8];
          nibbles_to_f32(y[k], f);
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            if ((gm >> h) & 1) {
              float sacc = acc[h][k];
#pragma unroll
              for (int j = 0; j < 8; ++j) sacc = __fmaf_rn(gv[h][j], f[j], sacc);
              acc[h][k] = sacc;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- optional side stream (fixed-width baselines): a byte per key, or
    // (meta_bits 4) two keys per byte, the even key in the low nibble
    const int64_t key0 = word * 32;
    if (S.meta) {
      const bool nib = S.meta_bits == 4;
      const uint8_t *mp = S.meta + (int64_t)g * (nib ? (n + 1) / 2 : n);
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        const int64_t i = key0 + k;
        const uint32_t v = i < n ? (nib ? (mp[i >> 1] >> (4 * (i & 1))) & 15u : mp[i]) : 0u;
        const float m = (float)v;
#pragma unroll
        for (int h = 0; h < GH; ++h) acc[h][k] = __fmaf_rn(S.meta_scale, m, acc[h][k]);
      }
    }

    // ---- logits ------------------------------------------------------------
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float *out = S.logits + (int64_t)(head_base + h) * S.ld + key0;
      if (S.vec_out && key0 + KPL <= n) {
#pragma unroll
        for (int k = 0; k < KPL; k += 4)
          *reinterpret_cast<float4 *>(out + k) =
              make_float4(acc[h][k], acc[h][k + 1], acc[h][k + 2], acc[h][k + 3]);
      } else {
#pragma unroll
        for (int k = 0; k < KPL; ++k)
          if (key0 + k < n) out[k] = acc[h][k];
      }
    }
  }
}

// ---- matrix-core scan (planes in HBM) --------------------------------------
// The contraction s_hi = C_h + sum_slot gamma_{h,slot} m_{slot,i} runs on
// v_mfma_i32_16x16x64_i8 (rows: 4 heads x 4 limbs, columns: 16 keys, K: 64
// slots = one pass).  Per head, gamma is put in fixed point
// G = rint(gamma 2^(30-E_h)) with 2^(E_h-1) <= max|gamma| < 2^E_h, and G is
// split into four balanced signed 8-bit limbs, so the integer products and
// sums of a pass are exact; the quantisation error is at most
// 2^-31 max|gamma| per weight, i.e. below 15 * 512 * 2^-31 * max|gamma| <=
// 1.2e-7 A_h.  Per pass, an fp32 step combines the limbs and adds
// 2^(E_h-30) times them to the key's running value, which starts at C_h (one
// rounding per pass).
//
// One 1024-thread block per CU (one round of resident blocks) over 2048-key
// tiles; an item is one pass (64 slots) of one tile.  Its 16 waves split into
// 8 producers and 8 consumers that pass items through two code buffers in LDS,
// with counters instead of block barriers (a block barrier made the waves that
// finished first wait for the slowest every step).
//  * Producers: a task is one slot group (8 slots x 4 planes = 32 rows) of one
//    tile, read with 16-byte loads: a quarter of the wave (16 lanes) covers one
//    row, 4 words per lane, and one load instruction covers the 4 planes of
//    one slot.  Tasks go round-robin to the 8 producer waves, each keeping two
//    in flight.  Two lane swaps (32-lane halves, then 16-lane rows) regroup the
//    words so that every lane holds one plane word (32 keys) of all 32 rows,
//    which it bit-transposes into 32 per-key nibble words in the item's buffer.
//  * Consumers: wave v runs the MFMAs for keys 256v .. 256v+255 of the item (16
//    blocks of 16 keys x 64 slots); its lanes end with 4 consecutive keys of
//    one head, written as one 16-byte store (or tested against the row's
//    threshold).  Consumers win issue arbitration: their phases set the pace.
// Wide loads matter: with 4-byte lanes the memory pipeline, not HBM, limits
// the read rate at this occupancy.
constexpr int kMThreads = 1024;                      // 8 producer + 8 consumer waves
constexpr int kMTileKeys = 2048;
constexpr int kPassGroups = 8;                        // 8 groups x 8 slots = K 64
constexpr int kMaxPasses = kMaxGroups / kPassGroups;  // 8
// group pitch in the code table: >= 2113 words (2048 keys + skews), = 1 mod 4
constexpr int kGroupPitch = 2113;
constexpr uint32_t kUnread = 0x80000000u;  // at or past the end of any kv head's planes

typedef int v4i __attribute__((ext_vector_type(4)));

// LDS index of (group-in-pass gp, key).  Skews: one word per 32 keys, two
// more per 1024 keys, and a pitch of 1 mod 4 between groups.  Transpose
// stores (32 lanes at keys 32w + t, w = 4m + k, k in {0,1} or {2,3}) and
// operand loads (16 lanes at keys 4n + e, two groups 2 apart) then hit 32
// distinct banks.
__device__ __forceinline__ int code_index(int gp, int key) {
  return gp * kGroupPitch + key + (key >> 5) + 2 * (key >> 10);
}

// The float t with (to_key(x) >= T) == (x >= t) for every finite x: T = 0
// keeps everything; keys above the largest finite one keep nothing.
__device__ __forceinline__ float key_threshold(uint32_t T) {
  if (T == 0) return -INFINITY;
  const float t = from_key(T);
  if (t != t) return T >= 0x80000000u ? INFINITY : -INFINITY;  // NaN patterns
  return t;
}

// ---- code-buffer ring between the waves of one block -------------------------
// Counters in LDS that only grow.  A wave signals once its own LDS accesses
// to the buffer are complete (lgkmcnt 0, then one LDS add by lane 0); a wave
// that waits spins, sleeping between reads, until the count reaches the
// target.  Every wave of the block takes part in every round, so the targets
// are always reached; the spin is capped all the same (~10^8 cycles), so no
// wave can wait forever.
constexpr uint32_t kRingSpinCap = 1u << 21;
#ifndef FATHOM_RING_SLEEP
#define FATHOM_RING_SLEEP 1
#endif

__device__ __forceinline__ void ring_wait(uint32_t *ctr, uint32_t target) {
  for (uint32_t spin = 0; spin < kRingSpinCap; ++spin) {
    const uint32_t v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (v >= target) break;
    __builtin_amdgcn_s_sleep(FATHOM_RING_SLEEP);
  }
  asm volatile("" ::: "memory");  // buffer accesses stay after the wait
}

__device__ __forceinline__ void ring_signal(uint32_t *ctr) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Lower bound on the high limb pair hi = a2 + 256*a3 of every key whose
// one-pass score s = fl(fl(fl(hi)*65536 + fl(lo))*scale + C) reaches tf
// (scale > 0, |hi|, |lo| < 2^26: each limb sum is below 64*128*15 < 2^17).
// s >= tf gives t*scale + C >= tf*(1 - 2^-23) - 2^-149 for t = fl(hi*65536 +
// lo), hence hi*65536 + lo >= (tf - C)/scale minus relative rounding terms
// of 2^-23 and the |lo| bound; all margins below are taken with room (2^-20
// relative, 2^27 absolute), and the result rounds down.  A key with hi below
// the bound cannot be a candidate.
__device__ __forceinline__ int hi_bound(float tf, float C, float scale) {
  if (tf == -INFINITY) return INT_MIN;
  if (tf == INFINITY) return INT_MAX;
  const double tfd = tf, Cd = C, sc = scale;
  const double rel = 9.5367431640625e-07;  // 2^-20
  double x = (tfd - Cd - rel * (fabs(tfd) + fabs(Cd))) / sc;
  x -= rel * fabs(x) + 134217728.0;        // + 2^27 for lo and the roundings
  const double h = floor(x / 65536.0) - 1.0;
  if (h <= (double)INT_MIN) return INT_MIN;
  if (h >= (double)INT_MAX) return INT_MAX;
  return (int)h;
}

// Group pre-check of a one-pass group candidate scan (one output row per kv
// head, scored by the fp32 logits of its GH query heads added in fp64 and
// rounded once).  The group score is linear in the codes: with Gamma_slot =
// sum_h gamma_h,slot in fixed point (scale 2^(EG-30), integer limbs as for
// the heads), every head's exact value C_h + scale_h * X_h adds up to
// sum_h C_h + gscale * XG plus at most gmarg, which covers the weights'
// rounding to the two fixed points (15 codes x nslots x half a unit of
// each) and every fp32 / fp64 rounding of the logits and of their sum
// (2^-20 of sum_h B_h, B_h = |C_h| + 15 nslots max|gamma_h|, plus 8 units of
// each scale).  A key whose group score reaches tf therefore has
// gscale * XG >= tf - sum C_h - gmarg; its high limb pair hiG = XG >> 16
// (|low part| < 2^26) is then at least group_bound.  Keys below it are no
// candidates.
__device__ __forceinline__ int group_bound(float tf, double sumC, double marg, float gscale) {
  if (tf == -INFINITY) return INT_MIN;
  if (tf == INFINITY) return INT_MAX;
  double x = ((double)tf - sumC - marg) / (double)gscale;
  x -= 134217728.0;  // 2^27: the low limb pair and slack
  const double h = floor(x / 65536.0) - 1.0;
  if (h <= (double)INT_MIN) return INT_MIN;
  if (h >= (double)INT_MAX) return INT_MAX;
  return (int)h;
}

// Where the candidate words of one lane go: positions pos, pos+1, ... of the
// scan block's segment of output row `row`, and past its end the row's
// overflow list, whose slots the lane takes with one global add for all of
// its overflowing words (top keys clustered in one stretch of the row send
// hundreds of words from one block; one atomic per word would serialise).
struct CandSink {
  uint64_t *seg;       // the block's segment of the row
  uint64_t *ovf;       // the row's overflow list
  uint32_t pos, cap;   // next segment position; segment capacity
  uint32_t obase;      // first overflow slot of this lane
};

__device__ __forceinline__ CandSink cand_sink(KScanSess &S, int row, int seg, uint32_t pos,
                                              uint32_t count) {
  CandSink c;
  c.seg = S.cand + (int64_t)row * kFusedCap + (int64_t)seg * S.seg_cap;
  c.ovf = S.ovf + (int64_t)row * kCandCap;
  c.pos = pos;
  c.cap = (uint32_t)S.seg_cap;
  const uint32_t in_seg = pos >= c.cap ? 0u : (c.cap - pos < count ? c.cap - pos : count);
  c.obase = 0;
  if (count > in_seg)
    c.obase = atomicAdd(&S.ovf_cnt[(int64_t)row * kCntStride], count - in_seg);
  return c;
}

__device__ __forceinline__ void cand_put(CandSink &c, uint64_t wd) {
  if (c.pos < c.cap) {
    c.seg[c.pos] = wd;
  } else {
    if (c.obase < (uint32_t)kCandCap) c.ovf[c.obase] = wd;
    ++c.obase;
  }
  ++c.pos;
}

// Set-up-only state of the matrix-core kernel, overlaid on its code table.
template <int GH>
struct MfmaSetup {
  SlotTable<GH> T;
  SlotScratch<GH> X;
};

// What the main loop of the matrix-core scan needs from its set-up, as one
// scan of a fused call stores it for the later ones.
struct alignas(16) SlotRecord {
  int32_t nslots, gvalid, pad[2];
  float C[kMaxGH], scale[kMaxGH];
  int16_t desc[kMaxSlots];
  int32_t limbs[kMaxPasses][64][4];
  // group pre-check (GroupCheck), when gvalid
  int32_t glimbs[64][4];
  double gsumC, gmarg;
  float gscale, gpad[3];
};

// Per-block ranges (BLK): gamma and C_h change with every 2048-key tile.  The
// block's set-up forms, for each of its tiles, delta_c,tile of every channel,
// C_h,tile (in the slot table's fp64 order) and the candidate bound, and one
// fixed-point exponent per head for all of its tiles, from the largest
// |gamma| over them (quantisation error <= 2^-31 of that per weight, still
// far inside the tolerance).  Every producer task, once its codes are
// stored, writes the int8 limbs of its 8 slots' gamma = q_hc * delta_c,tile
// beside them; consumers read those A operands with the codes, after the same
// fill wait.
constexpr int kBlkTiles = 16;  // tiles per block with per-block ranges (the launcher keeps to it)
struct alignas(16) ItemLimbs {
  int32_t limbs[64][4];  // A operands of the item's pass (layout of s_limbs)
};

// A fused final block inside the recompute scan's launch: output row
// blockIdx.x (final_rows per session) is ranked from its candidates, with
// the code buffers as its LDS; a row whose candidate count is out of range
// is recorded (row and kv head) and left to the scan blocks of its kv head,
// which apply the same rule to the same counts.
__device__ __forceinline__ void scan_final_block(KScanArgs &a, uint8_t *lds) {
  const int o = blockIdx.x;
  const int si = o / a.final_rows, r = o % a.final_rows;
  KScanSess &S = a.s[si];
  FinalScratch X;
  X.s = reinterpret_cast<uint64_t *>(lds);
  X.win = X.s + kCandCap;
  X.red = X.win + kBuckCap;
  X.hist = reinterpret_cast<int *>(X.red + kSelThreads / 64);
  X.above = X.hist + kRankBins;
  X.wave_tot = X.above + kRankBins + 1;
  X.s_res = X.wave_tot + 16;
  X.s_count = X.s_res + 2;
  X.s_off = X.s_count + 1;
  const int k = a.out_k;
  if (!fused_final_row(S.cand + (int64_t)r * kFusedCap, S.seg_cnt + (int64_t)r * kMaxSeg,
                       S.nseg, S.ovf + (int64_t)r * kCandCap, S.ovf_cnt + (int64_t)r * kCntStride,
                       S.n, k, S.out_idx + (int64_t)r * k, S.out_vals + (int64_t)r * k, X) &&
      threadIdx.x == 0) {
    S.row_flag[r] = 1;
    S.redo[r / max(1, a.final_rows / a.hkv)] = 1;
  }
}

// META: the sessions carry a side stream (its bytes are prefetched with the
// planes, which costs registers the other variants do not spend).
template <int GH, int MODE, bool META, bool BLK>
__global__ __launch_bounds__(kMThreads) void scan_mfma_kernel(ScanArgs a) {
  const BlockWork bw = block_work(a);
  KScanSess &S = *bw.S;
  const int g = bw.g, head_base = bw.head_base;
  const int64_t n = S.n;
  const int64_t W = S.W;
  __shared__ __align__(16) uint32_t s_codes[2][kPassGroups * kGroupPitch + 4];  // the ring's buffers
  static_assert(sizeof(MfmaSetup<GH>) <= sizeof(s_codes[0]), "set-up overlay");
  static_assert(kFinalScratchBytes <= sizeof(s_codes), "fused final overlay");
  __shared__ __align__(16) int32_t s_limbs[kMaxPasses][64][4];
  __shared__ __align__(16) int16_t s_desc[kMaxSlots];
  __shared__ float s_scale[kMaxGH], s_C[kMaxGH];
  __shared__ int s_exp[kMaxGH];
  __shared__ uint32_t s_segc[kMaxGH];  // candidates this block found per row
  __shared__ float s_tf[kMaxGH];       // float thresholds of the block's rows
  __shared__ int s_ht[kMaxGH];         // integer pre-check bounds (see hi_bound)
  __shared__ int s_nslots;
  // group pre-check: A operands of the group weights' limbs, its integer
  // bound, whether the block has it, and (set-up) the record's constants
  __shared__ __align__(16) typename std::conditional<!BLK && GH == kMaxGH, int32_t[64][4],
                                                      char>::type s_glimbs;
  __shared__ int s_gvalid, s_ght;
  __shared__ double s_gsumC, s_gmarg;
  __shared__ float s_gscale;
  __shared__ int s_last;  // recompute scan: this block finished its (kv head, chunk) last
  __shared__ uint32_t s_redo_rows;  // recompute scan: bit j = row j of the block's rows
  // code-buffer ring: [0..1] groups stored in buffer 0/1 (one count per
  // producer task), [2..3] releases (one per consumer wave and item); counts
  // only grow during a launch
  __shared__ uint32_t s_ring[4];
  // per-block ranges: the items' A operands, C_h and the candidate bound per
  // tile
  __shared__ typename std::conditional<BLK, ItemLimbs[2], char>::type s_hdr;
  __shared__ typename std::conditional<BLK, float[kBlkTiles][kMaxGH], char>::type s_tC;
  __shared__ typename std::conditional<BLK, float[kBlkTiles][kD], char>::type s_tD;
  __shared__ typename std::conditional<BLK && MODE == kScanCand, int[kBlkTiles][kMaxGH],
                                       char>::type s_tht;
  __shared__ uint32_t s_gmax[kMaxGH];
  // per-block ranges: q_hc of each slot's channel for the heads using the
  // slot, else 0 (in place of the per-layer limbs)
  float(*const s_gq)[kMaxGH] = reinterpret_cast<float(*)[kMaxGH]>(&s_limbs[0][0][0]);
  static_assert(sizeof(float) * kMaxSlots * kMaxGH <= sizeof(s_limbs), "slot weights overlay");
  const int tid = threadIdx.x;
  if constexpr (MODE == kScanLogits) {
    // recompute scan of a fused call: the fused final's blocks come first
    KScanArgs &ka = *(KScanArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    if ((int)blockIdx.x < ka.n_final) {
      scan_final_block(ka, reinterpret_cast<uint8_t *>(&s_codes[0][0]));
      return;
    }
    if (S.redo_done) {
      // The block's rows whose candidate count lies outside [k, kCandCap]
      // (the rows the final blocks leave unanswered, by the same rule); a
      // block with none returns at once.
      if (tid == 0) s_redo_rows = 0;
      __syncthreads();
      const int wv = tid >> 6, ln = tid & 63;
      if (wv < (a.out_group > 1 ? 1 : GH) && n > kCandCap) {
        const int row = a.out_group > 1 ? g : head_base + wv;
        uint32_t c = 0;
        for (int b = ln; b < S.nseg; b += 64) c += S.seg_cnt[(int64_t)row * kMaxSeg + b];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) c += (uint32_t)__shfl_xor((int)c, off);
        if (ln == 0 && (c < (uint32_t)a.out_k || c > (uint32_t)kCandCap))
          atomicOr(&s_redo_rows, 1u << wv);
      }
      __syncthreads();
      if (s_redo_rows == 0) return;
    }
  }
  // Work items = (tile, pass) of this block's tiles in order; item i goes
  // through code buffer i % 2.  Visited tile v of this block: all tiles, or
  // (sample mode) nvtiles tiles spread evenly over the ntiles real ones.
  const int tiles_per_block = S.tiles_per_block;
  const int nvtiles = S.nvtiles, ntiles_real = S.ntiles;
  auto real_tile = [&](int v) -> int {
    return MODE == kScanSample ? (int)sample_tile(v, nvtiles, ntiles_real) : v;
  };
  int ntiles = 0;
  while (ntiles < tiles_per_block && bw.tile0 + ntiles * bw.tile_step < nvtiles) ++ntiles;
  // per-block ranges: wave w's first tile's lo and hi (channels lane, lane +
  // 64), loaded before the set-up so that their latency overlaps it
  float pf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (BLK) {
    const int wv = tid >> 6, ln = tid & 63;
    if (wv < ntiles) {
      const int64_t r0 = ((int64_t)g * S.rs + real_tile(bw.tile0 + wv * bw.tile_step)) * kD;
      pf[0] = S.lo[r0 + ln];
      pf[1] = S.lo[r0 + ln + 64];
      pf[2] = S.hi[r0 + ln];
      pf[3] = S.hi[r0 + ln + 64];
    }
  }
  SlotRecord *rec = S.table ? reinterpret_cast<SlotRecord *>(S.table) + bw.rec : nullptr;
  // candidate modes: the rows' threshold keys, loaded now so that their
  // latency overlaps the set-up's own loads
  uint32_t thr_key = 0;
  if constexpr (MODE == kScanCand)
    if (tid < GH) thr_key = S.thr[head_base + tid];
  if constexpr (MODE == kScanCandGroup)
    if (tid < GH) thr_key = S.thr[g];
  if constexpr (BLK) {
    // Slot order (from an earlier scan of the call, or built with unit
    // weights), q and t of the block's heads, per-slot weights s_gq; then per
    // tile delta_c, C_h and the heads' largest |gamma| (wave w takes tile w,
    // lanes channels lane and lane + 64).
    MfmaSetup<GH> &U = *reinterpret_cast<MfmaSetup<GH> *>(s_codes[0]);
    if (S.table_mode == kTableRead) {
      if (tid == 0) s_nslots = rec->nslots;
      constexpr int kDescVec = sizeof(rec->desc) / 16;
      if (tid < kDescVec)
        reinterpret_cast<int4 *>(s_desc)[tid] = reinterpret_cast<const int4 *>(rec->desc)[tid];
      for (int e = tid; e < GH * kD; e += kMThreads) {
        U.X.q[e / kD][e % kD] = S.q[(int64_t)(head_base + e / kD) * kD + e % kD];
        U.X.t[e / kD][e % kD] = S.plan[(int64_t)(head_base + e / kD) * kD + e % kD];
      }
    } else {
      build_slot_table<GH>(U.T, U.X, S, g, head_base);
      const int nslots = U.T.nslots;
      if (tid == 0) s_nslots = nslots;
      for (int e = tid; e < kMaxSlots; e += kMThreads)
        s_desc[e] = e < nslots ? U.T.desc[e] : (int16_t)0;
      if (S.table_mode == kTableWrite && bw.tile0 == 0) {
        // for the later scans of this call (one block per kv head stores it)
        if (tid == 0) rec->nslots = nslots;
        for (int e = tid; e < kMaxSlots; e += kMThreads)
          rec->desc[e] = e < nslots ? U.T.desc[e] : (int16_t)0;
      }
    }
    if (tid < kMaxGH) s_gmax[tid] = 0u;
    __syncthreads();
    const int nslots = s_nslots;
    for (int e = tid; e < kMaxSlots * GH; e += kMThreads) {
      const int slot = e / GH, h = e % GH;
      const int desc = s_desc[slot];
      const int c = (desc >> 3) & (kD - 1), dep = desc & 7;
      s_gq[slot][h] = slot < nslots && U.X.t[h][c] >= dep ? U.X.q[h][c] : 0.0f;
    }
    const int wv = tid >> 6, ln = tid & 63;
    float m[GH];
#pragma unroll
    for (int j = 0; j < GH; ++j) m[j] = 0.0f;
    static_assert(kBlkTiles <= kMThreads / 64, "one tile per wave");
    if (wv < ntiles) {
      const int ti = wv;
      const float l0 = pf[0], l1 = pf[1];
      const float d0 = __fmul_rn(__fsub_rn(pf[2], l0), 0.0625f);
      const float d1 = __fmul_rn(__fsub_rn(pf[3], l1), 0.0625f);
      s_tD[ti][ln] = d0;
      s_tD[ti][ln + 64] = d1;
#pragma unroll
      for (int j = 0; j < GH; ++j) {
        const int t0 = U.X.t[j][ln], t1 = U.X.t[j][ln + 64];
        const float q0 = U.X.q[j][ln], q1 = U.X.q[j][ln + 64];
        if (t0 > 0) m[j] = fmaxf(m[j], fabsf(__fmul_rn(q0, d0)));
        if (t1 > 0) m[j] = fmaxf(m[j], fabsf(__fmul_rn(q1, d1)));
        double v0 = (double)q0 * ((double)l0 + (double)d0 * (double)(1 << (4 - t0)) * 0.5);
        double v1 = (double)q1 * ((double)l1 + (double)d1 * (double)(1 << (4 - t1)) * 0.5);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          v0 = __dadd_rn(v0, __shfl_xor(v0, off));
          v1 = __dadd_rn(v1, __shfl_xor(v1, off));
        }
        if (ln == 0) s_tC[ti][j] = (float)__dadd_rn(v0, v1);
      }
    }
#pragma unroll
    for (int j = 0; j < GH; ++j) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m[j] = fmaxf(m[j], __shfl_xor(m[j], off));
      if (ln == 0) atomicMax(&s_gmax[j], __float_as_uint(m[j]));
    }
    __syncthreads();
    // one fixed-point exponent per head for the block's tiles
    if (tid < GH) {
      const float mx = __uint_as_float(s_gmax[tid]);
      int e = 0;
      if (mx > 0.0f) frexpf(mx, &e);
      s_exp[tid] = e;
      s_scale[tid] = ldexpf(1.0f, e - 30);
    }
  } else if (S.table_mode == kTableRead) {
    // the set-up an earlier scan of this call stored
    if (tid == 0) s_nslots = rec->nslots;
    if (tid < GH) {
      s_scale[tid] = rec->scale[tid];
      s_C[tid] = rec->C[tid];
    }
    constexpr int kDescVec = sizeof(rec->desc) / 16, kLimbVec = sizeof(rec->limbs) / 16;
    if (tid < kDescVec)
      reinterpret_cast<int4 *>(s_desc)[tid] = reinterpret_cast<const int4 *>(rec->desc)[tid];
    for (int e = tid; e < kLimbVec; e += kMThreads)
      reinterpret_cast<int4 *>(&s_limbs[0][0][0])[e] =
          reinterpret_cast<const int4 *>(&rec->limbs[0][0][0])[e];
    if constexpr (MODE == kScanCandGroup && !BLK && GH == kMaxGH) {
      if (tid == 0) {
        s_gvalid = rec->gvalid;
        s_gsumC = rec->gsumC;
        s_gmarg = rec->gmarg;
        s_gscale = rec->gscale;
      }
      if (tid < 64)
        reinterpret_cast<int4 *>(&s_glimbs[0][0])[tid] =
            reinterpret_cast<const int4 *>(&rec->glimbs[0][0])[tid];
    }
  } else {
    MfmaSetup<GH> &U = *reinterpret_cast<MfmaSetup<GH> *>(s_codes[0]);
    SlotTable<GH> &T = U.T;
    build_slot_table<GH>(T, U.X, S, g, head_base);
    const int nslots = T.nslots;
    const int ngroups = (nslots + 7) >> 3;
    const int npasses = max(1, (ngroups + kPassGroups - 1) / kPassGroups);
    // fixed-point exponent per head
    if (tid < GH) {
      const float m = __uint_as_float(T.gmax[tid]);
      int e = 0;
      if (m > 0.0f) frexpf(m, &e);
      s_exp[tid] = e;
      s_scale[tid] = ldexpf(1.0f, e - 30);
      s_C[tid] = T.C[tid];
    }
    if (tid == 0) s_nslots = nslots;
    for (int e = tid; e < npasses * kPassGroups * 8; e += kMThreads)
      s_desc[e] = e < nslots ? T.desc[e] : (int16_t)0;
    __syncthreads();
    // A operands: lane l = row (head (l%16)/4, limb (l%16)%4), slot chunk l/16;
    // dword d, byte b <-> slot 64p + 16(l/16) + 8(d/2) + 2b + (d%2), the order
    // in which the code words are split into bytes below.
    uint8_t *limb_bytes = reinterpret_cast<uint8_t *>(&s_limbs[0][0][0]);
    for (int idx = tid; idx < npasses * 64 * 16; idx += kMThreads) {
      const int p = idx >> 10, l = (idx >> 4) & 63, d = (idx >> 2) & 3, b = idx & 3;
      const int r = l & 15, h = r >> 2, limb = r & 3, j = l >> 4;
      const int slot = 64 * p + 16 * j + 8 * (d >> 1) + 2 * b + (d & 1);
      int v = 0;
      if (h < GH && slot < nslots) {
        int G = (int)rintf(ldexpf(T.gam[slot][h], 30 - s_exp[h]));
        for (int i = 0; i < limb; ++i) {
          const int dg = ((G + 128) & 255) - 128;
          G = (G - dg) >> 8;
        }
        v = ((G + 128) & 255) - 128;
      }
      limb_bytes[idx] = (uint8_t)(int8_t)v;
    }
    if constexpr (!BLK && GH == kMaxGH) {
      // Group pre-check of a one-pass call scored per GQA group: Gamma_slot =
      // sum_h gamma_h,slot (fp64, exact) in fixed point below 2^30, its limbs
      // in the A layout above (every row block holds them), and the margin.
      const bool gbuild = a.out_group > 1 && npasses == 1;  // block-uniform
      if (tid == 0) s_gvalid = gbuild ? 1 : 0;
      if (gbuild) {
        // |Gamma_slot| <= sum_h max |gamma_h| < 2^eg: the exponent needs no
        // pass over the slots
        double gsum = 0.0;
#pragma unroll
        for (int h = 0; h < GH; ++h) gsum += (double)__uint_as_float(T.gmax[h]);
        int eg = 0;
        if (gsum > 0.0) frexp(gsum * (1.0 + 1.0e-12), &eg);  // (rounded up past the sum)
        const double to_fixed = __longlong_as_double((long long)(30 - eg + 1023) << 52);
        uint8_t *gl = reinterpret_cast<uint8_t *>(&s_glimbs[0][0]);
        for (int idx = tid; idx < 64 * 16; idx += kMThreads) {
          const int l = idx >> 4, d = (idx >> 2) & 3, b = idx & 3;
          const int limb = (l & 15) & 3, j = l >> 4;
          const int slot = 16 * j + 8 * (d >> 1) + 2 * b + (d & 1);
          int v = 0;
          if (slot < nslots) {
            double gs = 0.0;
#pragma unroll
            for (int h = 0; h < GH; ++h) gs = __dadd_rn(gs, (double)T.gam[slot][h]);
            int G = (int)rint(gs * to_fixed);
            for (int i = 0; i < limb; ++i) {
              const int dg = ((G + 128) & 255) - 128;
              G = (G - dg) >> 8;
            }
            v = ((G + 128) & 255) - 128;
          }
          gl[idx] = (uint8_t)(int8_t)v;
        }
        if (tid == 0) {
          // half a fixed-point unit of every head and of Gamma: 2^(e - 31)
          double sumC = 0.0, sumB = 0.0, sumS = 0.0;
          double half = __longlong_as_double((long long)(eg - 31 + 1023) << 52);
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            const double ch = (double)s_C[h];
            sumC += ch;
            sumB += fabs(ch) + 15.0 * nslots * (double)__uint_as_float(T.gmax[h]);
            sumS += (double)s_scale[h];
            half += __longlong_as_double((long long)(s_exp[h] - 31 + 1023) << 52);
          }
          s_gsumC = sumC;
          s_gmarg = 9.5367431640625e-07 * sumB + 8.0 * sumS + 15.0 * nslots * half;
          s_gscale = ldexpf(1.0f, eg - 30);
        }
      }
    }
  }
  if (tid < 4) s_ring[tid] = 0u;
  if (tid < GH) {
    s_segc[tid] = 0;
    if constexpr (MODE == kScanCand) {
      s_tf[tid] = key_threshold(thr_key);
      if (!BLK) s_ht[tid] = hi_bound(s_tf[tid], s_C[tid], s_scale[tid]);
    }
    if constexpr (MODE == kScanCandGroup) s_tf[tid] = key_threshold(thr_key);
  }
  if constexpr (MODE == kScanCandGroup && !BLK && GH == kMaxGH)
    if (tid == 0 && s_gvalid)
      s_ght = group_bound(key_threshold(thr_key), s_gsumC, s_gmarg, s_gscale);
  __syncthreads();  // the code table is free from here on
  if constexpr (BLK && MODE == kScanCand) {
    // integer candidate bound of each tile and head
    for (int e = tid; e < ntiles * GH; e += kMThreads)
      s_tht[e / GH][e % GH] = hi_bound(s_tf[e % GH], s_tC[e / GH][e % GH], s_scale[e % GH]);
    __syncthreads();
  }
  const int nslots = s_nslots;
  // per-block ranges: at least one slot group (padding slots read nothing),
  // whose producer task writes each item's header
  const int ngroups = max(BLK ? 1 : 0, (nslots + 7) >> 3);
  // at least one pass, so that a plan reading nothing still writes C_h
  const int npasses = max(1, (ngroups + kPassGroups - 1) / kPassGroups);
  if (!BLK && S.table_mode == kTableWrite && bw.tile0 == 0) {
    // for the later scans of this call (one block per kv head stores it)
    if (tid == 0) rec->nslots = nslots;
    if (tid < GH) {
      rec->scale[tid] = s_scale[tid];
      rec->C[tid] = s_C[tid];
    }
    constexpr int kDescVec = sizeof(rec->desc) / 16;
    if (tid < kDescVec)
      reinterpret_cast<int4 *>(rec->desc)[tid] = reinterpret_cast<const int4 *>(s_desc)[tid];
    for (int e = tid; e < npasses * 64; e += kMThreads)
      reinterpret_cast<int4 *>(&rec->limbs[0][0][0])[e] =
          reinterpret_cast<const int4 *>(&s_limbs[0][0][0])[e];
    if constexpr (GH == kMaxGH && !BLK) {
      if (tid == 0) {
        rec->gvalid = s_gvalid;
        rec->gsumC = s_gsumC;
        rec->gmarg = s_gmarg;
        rec->gscale = s_gscale;
      }
      if (tid < 64 && s_gvalid)
        reinterpret_cast<int4 *>(&rec->glimbs[0][0])[tid] =
            reinterpret_cast<const int4 *>(&s_glimbs[0][0])[tid];
    } else {
      if (tid == 0) rec->gvalid = 0;
    }
  }

  // role 0: producer waves (load, regroup, transpose into a code buffer);
  // role 1: consumer waves (matrix cores over the buffer, epilogue).  wave =
  // index within the role.
  const int role = tid >> 9, wave = (tid >> 6) & 7, lane = tid & 63;
  const int quarter = lane >> 4, m16 = lane & 15;
  const int hh = lane >> 4;  // head of this lane's results (MFMA row block)
  const float Ch = !BLK && hh < GH ? s_C[hh] : 0.0f;
  const float scale = hh < GH ? s_scale[hh] : 0.0f;
  const uint32_t *gplanes = S.planes + (int64_t)g * kD * kPlanes * W;
  const int64_t ld = S.ld;
  // side stream: a byte per key, or (meta_bits 4) two keys per byte, the
  // even key in the low nibble
  const bool meta_nib = META && S.meta_bits == 4;
  const uint8_t *meta =
      META && S.meta ? S.meta + (int64_t)g * (meta_nib ? (n + 1) / 2 : n) : nullptr;
  const float meta_scale = S.meta_scale;
  float *out_row = hh < GH ? S.logits + (int64_t)(head_base + hh) * ld : nullptr;
  const bool vec_out = S.vec_out != 0;
  // One buffer resource over this kv head's planes (the launcher keeps them
  // within 2 GiB).  Plane slot s of channel c, word w sits at byte
  // c*chan_bytes + s*row_bytes + 4w; offsets at or past kUnread read 0 and
  // touch no memory, which is how unread planes are skipped.
  const uint32_t row_bytes = (uint32_t)(W * 4);
  const uint32_t chan_bytes = row_bytes * kPlanes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(gplanes), (short)0, (int32_t)(chan_bytes * kD), kRsrcWord3);
  // quarter k loads code bit k, i.e. plane slot 3 - k, words 4*m16 .. +3
  const uint32_t plane_sl = 3u - (uint32_t)quarter;
  const uint32_t lane_part = plane_sl * row_bytes + (uint32_t)m16 * 16u;

  const int nitems = ntiles * npasses;

  // float threshold of this lane's output row (candidate modes)
  const float row_tf = (MODE == kScanCand || MODE == kScanCandGroup) && hh < GH ? s_tf[hh] : 0.0f;
  // side stream: 4 aligned bytes per beta when rows start on 4-byte bounds
  // (4 keys per load: 4 bytes, or 2 bytes of nibbles)
  const bool meta_words = META && meta &&
                          ((reinterpret_cast<uintptr_t>(S.meta) & (meta_nib ? 1 : 3)) == 0) &&
                          (n & 3) == 0;
  const uint32_t meta_sh = meta_nib ? 4u : 8u, meta_mask = meta_nib ? 15u : 255u;

  if (role == 0) {
    // ==== producers.  A task is one slot group of one tile: 32 plane rows
    // (8 slots x 4 planes) read with 16-byte loads, regrouped, transposed and
    // stored in the code buffer of its item (tile, pass = group / 8).  The
    // ntiles * ngroups tasks go round-robin to the 8 producer waves, so that
    // all of them keep loads in flight whatever the group count; each wave
    // has two tasks in flight.
    const int ntasks = ntiles * ngroups;
    // Every call issues its 8 loads, also for a task past the last (their
    // offsets lie past the buffer: they read 0 and touch no memory), so that
    // the loads of the two tasks in flight always complete in issue order
    // and the wait for the older one leaves the newer one in flight.
    auto issue = [&](int k, uint32_t(&x)[32], uint32_t(&rr)[4]) {
      const bool live = k < ntasks;  // wave-uniform
      const int ti = live ? k / ngroups : 0;
      const int grp = live ? k - ti * ngroups : 0;
      const uint32_t tile = live ? (uint32_t)real_tile(bw.tile0 + ti * bw.tile_step) : 0u;
      const uint32_t tile_off = tile * (kMTileKeys / 8);
      const uint4 dv = *reinterpret_cast<const uint4 *>(&s_desc[grp * 8]);
      const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
      if constexpr (BLK) {
        // the channels of this lane's two limb slots (slots 2 (lane / 16)
        // and + 1 of the group; see item_limbs)
        const uint32_t dl = (lane >> 4) == 0 ? dw[0] : (lane >> 4) == 1 ? dw[1]
                          : (lane >> 4) == 2 ? dw[2] : dw[3];
        rr[0] = (dl >> 3) & (kD - 1);
        rr[1] = (dl >> 19) & (kD - 1);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t desc =
            __builtin_amdgcn_readfirstlane((dw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        const uint32_t c = (desc >> 3) & (kD - 1), dep = desc & 7u, top = desc >> 10;
        const uint32_t voff = live && plane_sl < dep && plane_sl >= top
                                  ? c * chan_bytes + tile_off + lane_part
                                  : kUnread;
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int32_t)voff, 0, 0);
        x[4 * i + 0] = (uint32_t)v[0];
        x[4 * i + 1] = (uint32_t)v[1];
        x[4 * i + 2] = (uint32_t)v[2];
        x[4 * i + 3] = (uint32_t)v[3];
      }
    };
    // per-block ranges: the A-operand bytes of slot group gp (of the npg
    // groups of pass p) for the block's tile ti.  Lane: row r = lane % 16
    // (head r / 4, limb r % 4) of the group's slots 2 (lane / 16) and + 1,
    // whose channels are rr[0], rr[1]; byte of (row, slot sl of the pass) in
    // the operands: lane 16 (sl / 16) + row, dword 2 ((sl % 16) / 8) +
    // sl % 2, byte (sl % 8) / 2.  The first group also clears the bytes of
    // groups the pass lacks.
    auto item_limbs = [&](int ti, int p, int gp, int npg, ItemLimbs &H, const uint32_t(&rr)[4]) {
      if constexpr (BLK) {
        const int r = lane & 15, ha = r >> 2, limb = r & 3;
        const int ea = s_exp[ha < GH ? ha : 0];
        uint8_t *lb = reinterpret_cast<uint8_t *>(&H.limbs[0][0]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int sl = 8 * gp + 2 * (lane >> 4) + u;
          const int slot = 64 * p + sl;
          const float gq = ha < GH ? s_gq[slot][ha] : 0.0f;  // 0: head does not use the slot
          int v = 0;
          if (gq != 0.0f) {
            int G = (int)rintf(ldexpf(__fmul_rn(gq, s_tD[ti][rr[u]]), 30 - ea));
            for (int i = 0; i < limb; ++i) {
              const int dg = ((G + 128) & 255) - 128;
              G = (G - dg) >> 8;
            }
            v = ((G + 128) & 255) - 128;
          }
          lb[((16 * (sl >> 4) + r) * 4 + 2 * ((sl & 15) >> 3) + (sl & 1)) * 4 + ((sl & 7) >> 1)] =
              (uint8_t)(int8_t)v;
        }
        if (gp == 0)
          for (int g2 = npg; g2 < kPassGroups; ++g2)
            if (lane < 32) H.limbs[16 * (g2 >> 1) + (lane & 15)][2 * (g2 & 1) + (lane >> 4)] = 0;
      }
    };
    // regroup and transpose task k's words in place and store them in its
    // item's code buffer, once the consumers have released that buffer
    auto produce = [&](int k, uint32_t(&x)[32], const uint32_t(&rr)[4]) {
      const int ti = k / ngroups, grp = k - ti * ngroups;
      const int item = ti * npasses + (grp >> 3);
      const int b = item & 1;
      ring_wait(&s_ring[2 + b], 8u * (uint32_t)(item >> 1));  // buffer free
      // quarter k ends with word 4*m16 + k of the 4 plane rows of every
      // slot: 32-lane halves first, then 16-lane rows
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto h02 = __builtin_amdgcn_permlane32_swap(x[4 * i + 0], x[4 * i + 2], false, false);
        const auto h13 = __builtin_amdgcn_permlane32_swap(x[4 * i + 1], x[4 * i + 3], false, false);
        x[4 * i + 0] = h02[0];
        x[4 * i + 2] = h02[1];
        x[4 * i + 1] = h13[0];
        x[4 * i + 3] = h13[1];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto r01 = __builtin_amdgcn_permlane16_swap(x[4 * i + 0], x[4 * i + 1], false, false);
        const auto r23 = __builtin_amdgcn_permlane16_swap(x[4 * i + 2], x[4 * i + 3], false, false);
        x[4 * i + 0] = r01[0];
        x[4 * i + 1] = r01[1];
        x[4 * i + 2] = r23[0];
        x[4 * i + 3] = r23[1];
      }
      // x[4j+q] = bit q of slot j for keys 32w..32w+31 of the tile,
      // w = 4*m16 + quarter; afterwards x[t] = the 8 codes of key 32w+t
      transpose32_perm(x);
      const int w = 4 * m16 + quarter;
      uint32_t *dst = &s_codes[b][code_index(grp & 7, 32 * w)];
#pragma unroll
      for (int t = 0; t < 32; ++t) dst[t] = x[t];
      if constexpr (BLK)
        item_limbs(ti, grp >> 3, grp & 7, min(kPassGroups, ngroups - (grp & ~7)), s_hdr[b], rr);
      ring_signal(&s_ring[b]);  // one group of the buffer filled
    };
    uint32_t x0[32], x1[32], r0[4] = {0u, 0u, 0u, 0u}, r1[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < 32; ++r) x0[r] = x1[r] = 0;
    issue(wave, x0, r0);
    issue(wave + 8, x1, r1);
    for (int k = wave; k < ntasks; k += 16) {
      produce(k, x0, r0);
      issue(k + 16, x0, r0);
      if (k + 8 < ntasks) produce(k + 8, x1, r1);
      issue(k + 24, x1, r1);
    }
  } else {
    // ==== consumers: wave v multiplies keys 256v .. 256v+255 of every item
    // (16 MFMAs of 16 keys x 64 slots); block b = 4*beta + e covers keys
    // 64*beta + 4*n + e (n = lane % 16); each lane ends with 4 consecutive
    // keys of head hh per beta.
    const int j = lane >> 4, nn = lane & 15;
    // the consumers, whose matrix and epilogue phases set the pace, win
    // issue arbitration over the producers (whose loads run well ahead)
    __builtin_amdgcn_s_setprio(1);
    // group pre-check operands (one-pass group calls)
    v4i AG = v4i{0, 0, 0, 0};
    int ght = INT_MAX;
    bool gcheck = false;
    if constexpr (MODE == kScanCandGroup && !META && !BLK && GH == kMaxGH) {
      gcheck = s_gvalid != 0;
      if (gcheck) {
        const int4 ag = *reinterpret_cast<const int4 *>(&s_glimbs[lane][0]);
        AG = v4i{ag.x, ag.y, ag.z, ag.w};
        ght = s_ght;
      }
    }
    float s[16];
    uint32_t fill_target[2] = {0u, 0u};  // groups stored in each buffer so far
    for (int it = 0; it < nitems; ++it) {
      const int b = it & 1;
      const int ti = it / npasses, p = it - ti * npasses;
      fill_target[b] += (uint32_t)max(0, min(kPassGroups, ngroups - kPassGroups * p));
      const int vt = bw.tile0 + ti * bw.tile_step;
      const int64_t tile_key0 = (int64_t)real_tile(vt) * kMTileKeys;
      const bool last_pass = p == npasses - 1;
      // side-stream bytes of this wave's keys, loaded before the wait
      uint32_t mw[4] = {0u, 0u, 0u, 0u};
      if (META && meta_words && last_pass && hh < GH) {
        const int64_t kb0 = tile_key0 + 256 * wave + 4 * nn;
#pragma unroll
        for (int beta = 0; beta < 4; ++beta)
          if (kb0 + 64 * beta + 4 <= n)
            mw[beta] = meta_nib
                           ? (uint32_t)*reinterpret_cast<const uint16_t *>(meta + (kb0 + 64 * beta) / 2)
                           : *reinterpret_cast<const uint32_t *>(meta + kb0 + 64 * beta);
      }
      int4 av;
      if constexpr (!BLK) av = *reinterpret_cast<const int4 *>(&s_limbs[p][lane][0]);
      // per-block ranges: the tile's C_h and bound (the item's operands are
      // read after the fill wait, beside its codes)
      float Cit = Ch;
      const float sit = scale;
      int htit = INT_MAX;
      if constexpr (BLK) {
        if (hh < GH) {
          Cit = s_tC[ti][hh];
          if constexpr (MODE == kScanCand) htit = s_tht[ti][hh];
        }
      } else if (MODE == kScanCand && hh < GH) {
        htit = s_ht[hh];
      }
      ring_wait(&s_ring[b], fill_target[b]);  // every group of the item stored
      if constexpr (BLK) av = *reinterpret_cast<const int4 *>(&s_hdr[b].limbs[lane][0]);
      const v4i A = v4i{av.x, av.y, av.z, av.w};
      if (p == 0) {
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = Cit;
      }
      const uint32_t *codes = s_codes[b];
      if constexpr (MODE == kScanCandGroup && !META && !BLK && GH == kMaxGH) {
        if (npasses == 1 && gcheck) {
          // one pass, one row per kv head: the products of the group weights
          // first; a key's heads' products and its group score are formed only
          // where some lane's group high limb pair reaches the row's bound
          // (group_bound), which no candidate misses, and then exactly as in
          // the general path below (fp32 sum, fp64 near the threshold).  The
          // buffer is released after the tests (they may read it again).
          const int64_t kb = tile_key0 + 256 * wave + 4 * nn;  // + 64*beta + e
          const int64_t rem = n - kb;
          const int lim = rem > 256 ? 256 : (int)rem;
          auto operand = [&](int q) -> v4i {
            const int key = 256 * wave + 64 * (q >> 2) + 4 * nn + (q & 3);
            const uint32_t w0 = codes[code_index(2 * j, key)];
            const uint32_t w1 = codes[code_index(2 * j + 1, key)];
            return v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                       (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
          };
          v4i accg[16];
#pragma unroll
          for (int q = 0; q < 16; ++q)
            accg[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(AG, operand(q), v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int hig = accg[q][2] + accg[q][3] * 256;
            const bool maybe = hh == 0 && 64 * (q >> 2) + (q & 3) < lim && hig >= ght;
            if (__ballot(maybe) != 0ull) {
              // this lane's head's logit of the key, as the logits scan forms it
              const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, operand(q), v4i{0, 0, 0, 0},
                                                                    0, 0, 0);
              const int lo = acc[0] + acc[1] * 256;
              const int hi = acc[2] + acc[3] * 256;
              const float t = __fmaf_rn((float)hi, 65536.0f, (float)lo);
              const float sh = __fmaf_rn(t, sit, Cit);
              const uint32_t v = __float_as_uint(sh);
              const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
              const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
              const auto p48 = __builtin_amdgcn_permlane16_swap(p32[1], p32[1], false, false);
              const float s1 = __uint_as_float(p16[1]);
              const float s2 = __uint_as_float(p32[1]);
              const float s3 = __uint_as_float(p48[1]);
              float approx = sh, mag = fabsf(sh);
              if (GH > 1) { approx = __fadd_rn(approx, s1); mag = __fadd_rn(mag, fabsf(s1)); }
              if (GH > 2) { approx = __fadd_rn(approx, s2); mag = __fadd_rn(mag, fabsf(s2)); }
              if (GH > 3) { approx = __fadd_rn(approx, s3); mag = __fadd_rn(mag, fabsf(s3)); }
              const float margin = __fmaf_rn(mag, 4.76837158203125e-07f /* 2^-21 */,
                                             1.1754943508222875e-38f /* 2^-126 */);
              const bool near = maybe && __fadd_rn(approx, margin) >= row_tf;
              float gs = approx;
              if (__ballot(near) != 0ull) {
                double dacc = (double)sh;
                if (GH > 1) dacc = __dadd_rn(dacc, (double)s1);
                if (GH > 2) dacc = __dadd_rn(dacc, (double)s2);
                if (GH > 3) dacc = __dadd_rn(dacc, (double)s3);
                gs = (float)dacc;
              }
              if (maybe && gs >= row_tf) {
                // a candidate: the next place in this block's segment of the
                // kv head's row (few keys get here, one LDS add each)
                CandSink sink = cand_sink(S, g, bw.tile0, atomicAdd(&s_segc[0], 1u), 1u);
                cand_put(sink, compose(to_key(gs), kb + 64 * (q >> 2) + (q & 3)));
              }
            }
          }
          ring_signal(&s_ring[2 + b]);  // buffer read (by this wave)
          continue;
        }
      }
      if (MODE == kScanCand && !META && npasses == 1) {
        // one pass, one row per head: the exact score of a key is formed
        // only where some lane's high limb pair reaches the row's integer
        // bound (hi_bound), which no candidate misses; then the same fp32
        // steps as below decide it
        const int64_t kb = tile_key0 + 256 * wave + 4 * nn;  // + 64*beta + e
        const int64_t rem = n - kb;
        const int lim = hh < GH ? (rem > 256 ? 256 : (int)rem) : 0;
        const int ht = htit;
        // all 16 products first; the buffer is released once they are issued
        v4i acc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = 256 * wave + 64 * (q >> 2) + 4 * nn + (q & 3);
          const uint32_t w0 = codes[code_index(2 * j, key)];
          const uint32_t w1 = codes[code_index(2 * j + 1, key)];
          const v4i B = v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                            (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
          acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
        ring_signal(&s_ring[2 + b]);  // buffer read (by this wave)
        // key kb + 64*(q/4) + q%4 may be a candidate only if its high limb
        // pair reaches the bound; exact scores where some lane needs one
        uint32_t mask = 0;
        float sv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int hi = acc[q][2] + acc[q][3] * 256;
          const bool maybe = 64 * (q >> 2) + (q & 3) < lim && hi >= ht;
          sv[q] = 0.0f;
          if (__ballot(maybe) != 0ull) {
            const int lo = acc[q][0] + acc[q][1] * 256;
            const float t = __fmaf_rn((float)hi, 65536.0f, (float)lo);
            sv[q] = __fmaf_rn(t, sit, Cit);
            mask |= (uint32_t)(maybe && sv[q] >= row_tf) << q;
          }
        }
        if (mask) {
          // this block's segment of the row's candidate store
          const uint32_t c = (uint32_t)__popc(mask);
          CandSink sink = cand_sink(S, head_base + hh, bw.tile0, atomicAdd(&s_segc[hh], c), c);
          while (mask) {
            const int q = __ffs(mask) - 1;
            mask &= mask - 1;
            float v = sv[0];
#pragma unroll
            for (int u = 1; u < 16; ++u) v = q == u ? sv[u] : v;
            cand_put(sink, compose(to_key(v), kb + 64 * (q >> 2) + (q & 3)));
          }
        }
        continue;
      }
#pragma unroll
      for (int beta = 0; beta < 4; ++beta) {
        v4i acc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 256 * wave + 64 * beta + 4 * nn + e;
          const uint32_t w0 = codes[code_index(2 * j, key)];
          const uint32_t w1 = codes[code_index(2 * j + 1, key)];
          const v4i B = v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                            (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
          acc[e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // limb pairs combine exactly in int32 (|sum| < 2^29)
          const int lo = acc[e][0] + acc[e][1] * 256;
          const int hi = acc[e][2] + acc[e][3] * 256;
          const float t = __fmaf_rn((float)hi, 65536.0f, (float)lo);
          s[4 * beta + e] = __fmaf_rn(t, sit, s[4 * beta + e]);
        }
      }
      ring_signal(&s_ring[2 + b]);  // buffer read (by this wave)
      if (!last_pass) continue;

      // ---- epilogue: 4 consecutive keys of head hh per beta
      const int64_t kb = tile_key0 + 256 * wave + 4 * nn;  // + 64*beta + e
      if (META && meta_words && hh < GH) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          s[q] = __fmaf_rn(meta_scale, (float)((mw[q >> 2] >> (meta_sh * (q & 3))) & meta_mask),
                           s[q]);
      } else if (META && meta && hh < GH) {
        uint32_t mb[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t key = kb + 64 * (q >> 2) + (q & 3);
          mb[q] = key < n ? (meta_nib ? (meta[key >> 1] >> (4 * (key & 1))) & 15u : meta[key]) : 0u;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = __fmaf_rn(meta_scale, (float)mb[q], s[q]);
      }
      const bool wave_full = tile_key0 + 256 * (wave + 1) <= n;  // wave-uniform
      if constexpr (MODE == kScanLogits) {
        if (hh < GH) {
          float *op = out_row + kb;
          if (vec_out && wave_full) {
#pragma unroll
            for (int beta = 0; beta < 4; ++beta)
              *reinterpret_cast<float4 *>(op + 64 * beta) =
                  make_float4(s[4 * beta], s[4 * beta + 1], s[4 * beta + 2], s[4 * beta + 3]);
          } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int64_t off = 64 * (q >> 2) + (q & 3);
              if (kb + off < n) op[off] = s[q];
            }
          }
        }
      } else if constexpr (MODE == kScanSample) {
        // The threshold's subsample: this wave's keys 256 wave + 4 nn + e
        // (beta = 0: the first 64 of every 256 keys) as the top 16 bits of
        // their score keys, 0 past the end of the row, at vt * 512 of the
        // output row's subsample.  A group call (a row per kv head) stores
        // the group score: its heads' logits added in fp64 in head order,
        // rounded once (lanes of head 0 gather the others by lane-row swaps).
        const int G = a.out_group;
        float sv[4] = {s[0], s[1], s[2], s[3]};
        int orow = head_base + hh;
        bool writer = hh < GH;
        if (G > 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t v = __float_as_uint(s[e]);
            const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            const auto p48 = __builtin_amdgcn_permlane16_swap(p32[1], p32[1], false, false);
            double acc = (double)s[e];
            if (G > 1) acc = __dadd_rn(acc, (double)__uint_as_float(p16[1]));
            if (G > 2) acc = __dadd_rn(acc, (double)__uint_as_float(p32[1]));
            if (G > 3) acc = __dadd_rn(acc, (double)__uint_as_float(p48[1]));
            sv[e] = (float)acc;
          }
          orow = g;
          writer = hh == 0;
        }
        if (writer) {
          uint32_t k16[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) k16[e] = kb + e < n ? to_key(sv[e]) >> 16 : 0u;
          uint16_t *op = S.sample + (int64_t)orow * kSubKeys + (int64_t)vt * kSampleSub +
                         64 * wave + 4 * nn;
          *reinterpret_cast<uint2 *>(op) = make_uint2(k16[0] | (k16[1] << 16), k16[2] | (k16[3] << 16));
        }
      } else {
        // candidates: score key at or above the row's threshold
        bool lane_rows = hh < GH;
        int row = head_base + hh;
        if constexpr (MODE == kScanCandGroup) {
          // group score: the group's fp32 logits added in fp64 in head order,
          // rounded once; lanes of head 0 hold the key's sum.  An fp32 sum
          // first: its error plus the final rounding stay below
          // 8 * 2^-24 * sum |s_h| (+ 2^-126 near zero), so a key whose fp32
          // sum misses the threshold by more than that is no candidate, and
          // the exact sum is formed only when some lane of the wave is
          // within that margin (every other lane's value is never used)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            // rows of 16 lanes are heads; row 0 receives rows 1, 2, 3 by
            // lane-row swaps (VALU, no LDS round trip)
            const uint32_t v = __float_as_uint(s[q]);
            const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            const auto p48 = __builtin_amdgcn_permlane16_swap(p32[1], p32[1], false, false);
            const float s1 = __uint_as_float(p16[1]);
            const float s2 = __uint_as_float(p32[1]);
            const float s3 = __uint_as_float(p48[1]);
            float approx = s[q], mag = fabsf(s[q]);
            if (GH > 1) { approx = __fadd_rn(approx, s1); mag = __fadd_rn(mag, fabsf(s1)); }
            if (GH > 2) { approx = __fadd_rn(approx, s2); mag = __fadd_rn(mag, fabsf(s2)); }
            if (GH > 3) { approx = __fadd_rn(approx, s3); mag = __fadd_rn(mag, fabsf(s3)); }
            const float margin = __fmaf_rn(mag, 4.76837158203125e-07f /* 2^-21 */,
                                           1.1754943508222875e-38f /* 2^-126 */);
            const bool near = hh == 0 && __fadd_rn(approx, margin) >= row_tf;
            if (__ballot(near) != 0ull) {
              double acc = (double)s[q];
              if (GH > 1) acc = __dadd_rn(acc, (double)s1);
              if (GH > 2) acc = __dadd_rn(acc, (double)s2);
              if (GH > 3) acc = __dadd_rn(acc, (double)s3);
              s[q] = (float)acc;
            } else {
              s[q] = approx;
            }
          }
          lane_rows = hh == 0;
          row = g;
        }
        // most waves hold no candidate at all: one max per lane and a ballot
        // decide whether the per-key tests run
        float mx = s[0];
#pragma unroll
        for (int q = 1; q < 16; ++q) mx = fmaxf(mx, s[q]);
        if (__ballot(lane_rows && mx >= row_tf) != 0ull && lane_rows) {
          // s >= t as floats is to_key(s) >= T (see key_threshold); keys
          // kb + 64*beta + e are valid while 64*beta + e < lim
          const int64_t rem = n - kb;
          const int lim = rem > 256 ? 256 : (int)rem;
          uint32_t mask = 0;
#pragma unroll
          for (int q = 0; q < 16; ++q)
            mask |= (uint32_t)((64 * (q >> 2) + (q & 3) < lim) && s[q] >= row_tf) << q;
          if (mask) {
            // this block's segment of the row's candidate store
            const uint32_t c = (uint32_t)__popc(mask);
            CandSink sink = cand_sink(
                S, row, bw.tile0, atomicAdd(&s_segc[MODE == kScanCandGroup ? 0 : hh], c), c);
            while (mask) {
              const int q = __ffs(mask) - 1;
              mask &= mask - 1;
              float v = s[0];
#pragma unroll
              for (int u = 1; u < 16; ++u) v = q == u ? s[u] : v;
              cand_put(sink, compose(to_key(v), kb + 64 * (q >> 2) + (q & 3)));
            }
          }
        }
      }
    }
  }
  if constexpr (MODE == kScanLogits) {
    // Recompute scan of a fused call: the block of a flagged (kv head, head
    // chunk) that finishes last ranks the chunk's flagged rows from the
    // logits every block of it wrote (a device-scope fence on each side of
    // the count makes those stores visible to it), in the code buffers.
    if (S.redo_done) {
      __syncthreads();
      if (tid == 0) {
        __threadfence();
        s_last = atomicAdd(&S.redo_done[bw.rec], 1u) == (uint32_t)(S.blocks_per_head - 1);
      }
      __syncthreads();
      if (s_last) {
        __threadfence();
        constexpr int kSortWords = kBuckCap + 2 * FATHOM_MAX_K;
        uint8_t *lds = reinterpret_cast<uint8_t *>(&s_codes[0][0]);
        static_assert((kSortWords + kBuckCap) * 8 + 16 * 8 + (2 * kRankBins + 8) * 4 + 16 * 4 +
                              16 <= sizeof(s_codes),
                      "selection scratch");
        SelScratch X;
        X.s = reinterpret_cast<uint64_t *>(lds);
        X.win = X.s + kSortWords;
        X.red = X.win + kBuckCap;
        X.hist = reinterpret_cast<int *>(X.red + 16);
        X.above = X.hist + kRankBins;
        X.wave_tot = X.above + kRankBins + 4;
        X.s_res = X.wave_tot + 16;
        X.s_count = X.s_res + 2;
        const int k = a.out_k, G = a.out_group;
        if (G > 1) {
          // one row per kv head, scored by the sum of its G query heads
          if (s_redo_rows & 1u)
            exact_row_topk(S.logits + (int64_t)head_base * S.ld, S.ld, G, n, k,
                           S.out_idx + (int64_t)g * k, S.out_vals + (int64_t)g * k, X);
        } else {
          for (int j = 0; j < GH; ++j) {
            const int o = head_base + j;
            if ((s_redo_rows >> j) & 1u)
              exact_row_topk(S.logits + (int64_t)o * S.ld, S.ld, 1, n, k,
                             S.out_idx + (int64_t)o * k, S.out_vals + (int64_t)o * k, X);
          }
        }
      }
    }
  }
  if constexpr (MODE == kScanCand || MODE == kScanCandGroup) {
    // every block reports its count (above seg_cap: the rest is in the
    // row's overflow list)
    __syncthreads();
    const int rows = MODE == kScanCandGroup ? 1 : GH;
    if (tid < rows) {
      const int row = MODE == kScanCandGroup ? g : head_base + tid;
      S.seg_cnt[(int64_t)row * kMaxSeg + bw.tile0] = s_segc[tid];
    }
  }
}

// out[h][i][c] = floor(code_ic / 2^(4 - t_hc)): the planes as a query reads them.
__global__ __launch_bounds__(256) void read_prefixes_kernel(
    const uint32_t *__restrict__ planes, int64_t n, int64_t W, int32_t group,
    const uint8_t *__restrict__ plan, uint8_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int c = threadIdx.x & 127;
  const int h = blockIdx.y;
  if (i >= n) return;
  const int g = h / group;
  const int t = plan[(int64_t)h * kD + c];
  const uint32_t *pc = planes + ((int64_t)g * kD + c) * kPlanes * W + i / 32;
  int v = 0;
  for (int s = 0; s < t; ++s) v = (v << 1) | ((pc[s * W] >> (i % 32)) & 1u);
  out[((int64_t)h * n + i) * kD + c] = (uint8_t)v;
}

// The fp32 kernel reads with streaming (non-temporal) loads: the planes
// stream once per step.
constexpr int kHostAux = 2;
constexpr int kHostTileKeys = 32 * 64 * (kScanThreads / 64);

using ScanFn = void (*)(ScanArgs);

template <int AUX, bool BLK>
ScanFn pick(int GH) {
  switch (GH) {
    case 1: return scan_kernel<1, AUX, BLK>;
    case 2: return scan_kernel<2, AUX, BLK>;
    case 3: return scan_kernel<3, AUX, BLK>;
    default: return scan_kernel<4, AUX, BLK>;
  }
}

template <int MODE, bool META, bool BLK>
ScanFn pick_mfma_mode(int GH) {
  switch (GH) {
    case 1: return scan_mfma_kernel<1, MODE, META, BLK>;
    case 2: return scan_mfma_kernel<2, MODE, META, BLK>;
    case 3: return scan_mfma_kernel<3, MODE, META, BLK>;
    default: return scan_mfma_kernel<4, MODE, META, BLK>;
  }
}

template <bool META, bool BLK>
ScanFn pick_mfma_meta(int GH, int mode) {
  switch (mode) {
    case kScanSample: return pick_mfma_mode<kScanSample, META, BLK>(GH);
    case kScanCand: return pick_mfma_mode<kScanCand, META, BLK>(GH);
    case kScanCandGroup: return pick_mfma_mode<kScanCandGroup, META, BLK>(GH);
    default: return pick_mfma_mode<kScanLogits, META, BLK>(GH);
  }
}

// (per-block ranges come without a side stream: the launcher refuses both)
ScanFn pick_mfma(int GH, int mode, bool meta, bool blk) {
  if (blk) return pick_mfma_meta<false, true>(GH, mode);
  return meta ? pick_mfma_meta<true, false>(GH, mode) : pick_mfma_meta<false, false>(GH, mode);
}

// Pinned-host planes: the link is the bound, the fp32 kernel with whole-word
// lanes keeps 256-byte wave accesses.  HBM planes: the matrix-core kernel
// (the fp32 kernel above 2^25 keys per session).
ScanFn kernel_for(bool host, int GH, int mode, bool meta, bool blk) {
  if (host) return blk ? pick<kHostAux, true>(GH) : pick<kHostAux, false>(GH);
  return pick_mfma(GH, mode, meta, blk);
}
int threads_for(bool host) { return host ? kScanThreads : kMThreads; }

int resident_blocks_per_cu(bool host, int GH, int mode, bool meta, bool blk) {
  static int cached[2][kMaxGH + 1][4][2][2] = {};
  int &c = cached[host ? 1 : 0][GH][mode][meta ? 1 : 0][blk ? 1 : 0];
  if (c == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, kernel_for(host, GH, mode, meta, blk), threads_for(host), 0);
    c = (e == hipSuccess && nb > 0) ? nb : 1;
  }
  return c;
}

// Residency of the sessions' planes; false (error set) if some are neither
// device nor pinned host memory.
bool planes_residency(const ScanSession *sess, int32_t n_sess, bool *any_host) {
  *any_host = false;
  for (int32_t j = 0; j < n_sess; ++j) {
    if (sess[j].residency != 0) {  // already resolved for this call
      *any_host |= sess[j].residency == 2;
      continue;
    }
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, sess[j].planes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      set_error("scan: planes of session %d are neither device nor pinned host memory", j);
      return false;
    }
    *any_host |= attr.type == hipMemoryTypeHost;
  }
  return true;
}

// The matrix-core kernel addresses a kv head's planes with 32-bit buffer
// offsets: plane rows of up to 2^20 words, i.e. 2^25 keys (2 GiB of planes per
// kv head).
constexpr int64_t kMfmaMaxKeys = (int64_t)1 << 25;

}  // namespace

int64_t scan_table_bytes(int32_t hkv, int32_t hq) {
  const int32_t group = hq / hkv;
  return (int64_t)hkv * ((group + kMaxGH - 1) / kMaxGH) * (int64_t)sizeof(SlotRecord);
}

bool resolve_residency(ScanSession *sess, int32_t n_sess) {
  for (int32_t j = 0; j < n_sess; ++j) {
    bool host = false;
    if (!planes_residency(&sess[j], 1, &host)) return false;
    sess[j].residency = host ? 2 : 1;
  }
  return true;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  int &c = cached[dev & 63];
  if (c == 0) {
    int ncu = 256;
    (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    c = ncu > 0 ? ncu : 256;
  }
  return c;
}

bool scan_can_fuse(const ScanSession *sess, int32_t n_sess) {
  bool any_host = false;
  if (!planes_residency(sess, n_sess, &any_host)) return false;
  for (int32_t j = 0; j < n_sess; ++j)
    if (sess_words(sess[j]) > plane_words(kMfmaMaxKeys)) return false;
  return !any_host;
}

int32_t launch_scan(const ScanSession *sess, int32_t n_sess, int32_t hkv, int32_t hq,
                    hipStream_t s, int32_t mode, int32_t *nseg_out, bool one_block_per_head,
                    int32_t final_rows) {
  const int32_t group = hq / hkv;
  const int ncu = device_cus();
  bool any_host = false;
  if (!planes_residency(sess, n_sess, &any_host)) return FATHOM_ERR_INVALID_ARG;
  int64_t max_w = 0;
  for (int32_t j = 0; j < n_sess; ++j) max_w = std::max(max_w, sess_words(sess[j]));
  const bool fp32_path = any_host || max_w > plane_words(kMfmaMaxKeys);
  if (fp32_path && mode != kScanLogits) {
    set_error("scan: sampled and candidate scans need device planes of at most 2^25 keys");
    return FATHOM_ERR_UNSUPPORTED;
  }
  if (mode == kScanCandGroup && group > kMaxGH) {
    set_error("scan: group candidate scans need hq/hkv <= %d", kMaxGH);
    return FATHOM_ERR_UNSUPPORTED;
  }
  for (int32_t j = 0; j < n_sess; ++j)
    if (fp32_path && (sess[j].redo_done || final_rows > 0)) {
      set_error("scan: recompute flags need the matrix-core scan");
      return FATHOM_ERR_UNSUPPORTED;
    }
  // per-block ranges: all sessions of a call or none, no side stream, and
  // each kv head's lo / hi rows within 2 GiB (32-bit buffer offsets)
  const bool blk = sess[0].rs > 0;
  for (int32_t j = 0; j < n_sess; ++j) {
    if ((sess[j].rs > 0) != blk || (blk && sess[j].meta)) {
      set_error("scan: per-block ranges need every session blocked and no side stream");
      return FATHOM_ERR_UNSUPPORTED;
    }
    if (blk && (sess[j].rs > ((int64_t)1 << 20) ||
                sess[j].rs * kBlockKeys < sess[j].n)) {
      set_error("scan: range stride %lld must cover the %lld keys' blocks, at most 2^20",
                (long long)sess[j].rs, (long long)sess[j].n);
      return FATHOM_ERR_INVALID_ARG;
    }
  }
  const bool cand = mode == kScanCand || mode == kScanCandGroup;
  const int64_t tile_keys =
      fp32_path ? (int64_t)kHostTileKeys : (int64_t)kMTileKeys;
  // tiles a session's blocks visit: all, or the sampled ones
  auto visited = [&](int64_t n) {
    const int64_t t = (n + tile_keys - 1) / tile_keys;
    return mode == kScanSample ? std::min<int64_t>(t, kSampleTiles) : t;
  };
  const int kernel_mode = fp32_path ? 0 : mode;
  bool any_meta = false;
  for (int32_t j = 0; j < n_sess; ++j) any_meta |= sess[j].meta != nullptr;
  for (int32_t s0 = 0; s0 < n_sess; s0 += kSessPerLaunch) {
    const int32_t cnt = std::min(kSessPerLaunch, n_sess - s0);
    // One tiling per session for all head chunks: one round of resident
    // blocks, every block taking the same number of tiles of one (session,
    // kv head) to amortise its plan set-up.
    int64_t total_tiles = 0;
    for (int j = 0; j < cnt; ++j) total_tiles += visited(sess[s0 + j].n) * hkv;
    const int64_t target_blocks =
        (int64_t)ncu *
        resident_blocks_per_cu(fp32_path, std::min(kMaxGH, group), kernel_mode, any_meta, blk);
    int64_t tpb_s[kSessPerLaunch];
    for (int j = 0; j < cnt; ++j) {
      const int64_t tiles = visited(sess[s0 + j].n);
      int64_t tpb = 1;
      if (one_block_per_head) tpb = std::max<int64_t>(1, tiles);
      if (total_tiles > target_blocks) tpb = std::max(tpb, (total_tiles + target_blocks - 1) / target_blocks);
      if (cand) tpb = std::max(tpb, (tiles + kMaxSeg - 1) / kMaxSeg);  // segments per row
      // per-block ranges: a block keeps C_h of each of its tiles in LDS (at
      // most 2^25 keys: 16 tiles per segment, within the cap)
      if (blk && !fp32_path) tpb = std::min<int64_t>(tpb, kBlkTiles);
      tpb_s[j] = std::max<int64_t>(1, std::min<int64_t>(tpb, tiles));
      if (nseg_out) nseg_out[s0 + j] = (int32_t)((tiles + tpb_s[j] - 1) / tpb_s[j]);
    }
    for (int32_t head0 = 0; head0 < group; head0 += kMaxGH) {
      const int GH = std::min(kMaxGH, group - head0);
      ScanArgs a{};
      a.n_sess = cnt;
      a.hkv = hkv;
      a.group = group;
      a.head0 = head0;
      a.out_k = sess[s0].out_k;
      a.out_group = sess[s0].out_group > 0 ? sess[s0].out_group : 1;
      // the fused final's blocks (first launch of the sessions only)
      a.final_rows = final_rows;
      a.n_final = mode == kScanLogits && head0 == 0 ? cnt * final_rows : 0;
      int32_t blocks = a.n_final;
      for (int j = 0; j < cnt; ++j) {
        const ScanSession &in = sess[s0 + j];
        ScanSess &o = a.s[j];
        o.planes = in.planes;
        o.lo = in.lo;
        o.hi = in.hi;
        o.q = in.q;
        o.plan = in.plan;
        o.meta = in.meta;
        o.logits = in.logits;
        o.n = in.n;
        o.W = sess_words(in);
        o.ld = in.ld;
        o.meta_scale = in.meta_scale;
        o.meta_bits = in.meta_bits == 4 ? 4 : 8;
        o.vec_out = ((reinterpret_cast<uintptr_t>(in.logits) & 15) == 0) && (in.ld % 4 == 0);
        o.sample = in.sample;
        o.thr = in.thr;
        o.cand = in.cand;
        o.seg_cnt = in.seg_cnt;
        o.ovf_cnt = in.ovf_cnt;
        o.ovf = in.ovf;
        o.redo = in.redo;
        o.redo_done = in.redo_done;
        o.row_flag = in.row_flag;
        o.nseg = in.nseg;
        o.out_idx = in.out_idx;
        o.out_vals = in.out_vals;
        o.rs = in.rs;
        o.table = fp32_path ? nullptr : in.table;
        o.table_mode = fp32_path || !in.table ? kTableNone : in.table_mode;
        const int64_t tiles = visited(in.n);
        o.nvtiles = (int32_t)tiles;
        o.ntiles = (int32_t)((in.n + tile_keys - 1) / tile_keys);
        o.tiles_per_block = (int32_t)tpb_s[j];
        o.blocks_per_head = (int32_t)((tiles + tpb_s[j] - 1) / tpb_s[j]);
        o.seg_cap = o.blocks_per_head > 0 ? kFusedCap / o.blocks_per_head : 0;
        o.block_begin = blocks;
        blocks += o.blocks_per_head * hkv;
      }
      if (blocks == 0) continue;
      hipLaunchKernelGGL(kernel_for(fp32_path, GH, mode, any_meta, blk), dim3(blocks),
                         dim3(threads_for(fp32_path)), 0, s, a);
      int32_t rc = hip_fail(hipGetLastError(), "scan launch");
      if (rc) return rc;
    }
  }
  return FATHOM_OK;
}

int32_t launch_read_prefixes(const uint32_t *planes, int64_t n, int32_t hkv,
                             const uint8_t *plan, int32_t hq, uint8_t *out,
                             hipStream_t s) {
  if (n == 0) return FATHOM_OK;
  hipLaunchKernelGGL(read_prefixes_kernel, dim3((unsigned)((n + 1) / 2), hq), dim3(256),
                     0, s, planes, n, plane_words(n), hq / hkv, plan, out);
  return hip_fail(hipGetLastError(), "read_prefixes launch");
}

}  // namespace fathom
