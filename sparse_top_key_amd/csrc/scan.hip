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
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMinSetupThreads = 256;             // smallest block building a slot table
constexpr int kMaxSlots = kD * kPlanes;           // (channel, depth) pairs
constexpr int kMaxGroups = kMaxSlots / 8;
constexpr int kMaxGH = 4;                          // heads per launch chunk

struct ScanSess {
  const uint32_t *planes;
  const float *lo, *hi, *q;
  const uint8_t *plan, *meta;
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
  float *sample;
  const uint32_t *thr;
  uint32_t *cnt;
  uint64_t *cand;
  uint32_t *seg_cnt;
  const uint32_t *redo;
  int32_t seg_cap;         // candidate words per (row, block) segment
  uint8_t *table;          // slot records of the session, or null
  int32_t table_mode;      // ScanTable
};

struct ScanArgs {
  ScanSess s[kSessPerLaunch];
  int32_t n_sess, hkv, group, head0;
};

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
// membership class, the per-head max |gamma| by LDS atomics.
template <int GH>
__device__ void build_slot_table(SlotTable<GH> &T, SlotScratch<GH> &X, KScanSess &S, int g,
                                 int head_base) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (tid < kD) {
    const int c = tid;
    const float lo = S.lo[g * kD + c];
    const float hi = S.hi[g * kD + c];
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

template <int GH, int AUX>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  const BlockWork bw = block_work(a);
  KScanSess &S = *bw.S;
  const int g = bw.g, tile0 = bw.tile0, tile_step = bw.tile_step, head_base = bw.head_base;
  const int64_t n = S.n;
  __shared__ SlotTable<GH> T;
  __shared__ SlotScratch<GH> X;
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
        for (int h = 0; h < GH; ++h) gv[h][j] = uniform_f(T.gam[grp * 8 + j][h]);
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

    // ---- optional 8-bit side stream (fixed-width baseline) ----------------
    const int64_t key0 = word * 32;
    if (S.meta) {
      const uint8_t *mp = S.meta + (int64_t)g * n + key0;
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        const float m = key0 + k < n ? (float)mp[k] : 0.0f;
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
// One 1024-thread block per CU (one round of resident blocks); its two halves
// of 8 waves each take one 2048-key tile (64 plane words per row) of an item,
// with a code table of their own, and run one step apart (a step lies
// between two barriers): while one half transposes an item, the other runs
// the matrix cores over its previous one.  In a pass, wave w of a half reads
// slot group w (8 slots x 4 planes = 32 rows) with 16-byte
// loads: a quarter of the wave (16 lanes) covers one row, 4 words per lane,
// and one load instruction covers the 4 planes of one slot.  Two lane swaps
// (32-lane halves, then 16-lane rows) regroup the words so that every lane
// holds one plane word (32 keys) of all 32 rows, which it bit-transposes into
// 32 per-key nibble words in LDS.  Then each wave runs the MFMAs for 256 keys
// (16 blocks of 16 keys); its lanes end with 4 consecutive keys of one head,
// written as one 16-byte store.  Wide loads matter: with 4-byte lanes the
// memory pipeline, not HBM, limits the read rate at this occupancy.
constexpr int kMThreads = 1024;                      // two halves of 8 waves
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

// Set-up-only state of the matrix-core kernel, overlaid on its code table.
template <int GH>
struct MfmaSetup {
  SlotTable<GH> T;
  SlotScratch<GH> X;
};

// What the main loop of the matrix-core scan needs from its set-up, as one
// scan of a fused call stores it for the later ones.
struct alignas(16) SlotRecord {
  int32_t nslots, pad[3];
  float C[kMaxGH], scale[kMaxGH];
  int16_t desc[kMaxSlots];
  int32_t limbs[kMaxPasses][64][4];
};

// META: the sessions carry a side stream (its bytes are prefetched with the
// planes, which costs registers the other variants do not spend).
template <int GH, int MODE, bool META>
__global__ __launch_bounds__(kMThreads) void scan_mfma_kernel(ScanArgs a) {
  const BlockWork bw = block_work(a);
  KScanSess &S = *bw.S;
  const int g = bw.g, head_base = bw.head_base;
  if (MODE == kScanLogits && S.redo && S.redo[g] == 0) return;  // kv head not flagged
  const int64_t n = S.n;
  const int64_t W = S.W;
  __shared__ __align__(16) uint32_t s_codes[2][kPassGroups * kGroupPitch + 4];  // per half
  static_assert(sizeof(MfmaSetup<GH>) <= sizeof(s_codes[0]), "set-up overlay");
  __shared__ __align__(16) int32_t s_limbs[kMaxPasses][64][4];
  __shared__ __align__(16) int16_t s_desc[kMaxSlots];
  __shared__ float s_scale[kMaxGH], s_C[kMaxGH];
  __shared__ int s_exp[kMaxGH];
  __shared__ uint32_t s_segc[kMaxGH];  // candidates this block found per row
  __shared__ float s_tf[kMaxGH];       // float thresholds of the block's rows
  __shared__ int s_nslots;
  const int tid = threadIdx.x;
  SlotRecord *rec = S.table ? reinterpret_cast<SlotRecord *>(S.table) + bw.rec : nullptr;
  if (S.table_mode == kTableRead) {
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
  }
  if (tid < GH) {
    s_segc[tid] = 0;
    // thresholds are read here, before any plane load is in flight
    if constexpr (MODE == kScanCand) s_tf[tid] = key_threshold(S.thr[head_base + tid]);
    if constexpr (MODE == kScanCandGroup) s_tf[tid] = key_threshold(S.thr[g]);
  }
  __syncthreads();  // the code table is free from here on
  const int nslots = s_nslots;
  const int ngroups = (nslots + 7) >> 3;
  // at least one pass, so that a plan reading nothing still writes C_h
  const int npasses = max(1, (ngroups + kPassGroups - 1) / kPassGroups);
  if (S.table_mode == kTableWrite && bw.tile0 == 0) {
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
  }

  // half = which of the block's two tiles of an item; wave = wave in the half
  const int half = tid >> 9, wave = (tid >> 6) & 7, lane = tid & 63;
  uint32_t *codes = s_codes[half];
  const int quarter = lane >> 4, m16 = lane & 15;
  const int hh = lane >> 4;  // head of this lane's results (MFMA row block)
  const float Ch = hh < GH ? s_C[hh] : 0.0f;
  const float scale = hh < GH ? s_scale[hh] : 0.0f;
  const uint32_t *gplanes = S.planes + (int64_t)g * kD * kPlanes * W;
  const int64_t ld = S.ld;
  const uint8_t *meta = META && S.meta ? S.meta + (int64_t)g * n : nullptr;
  const float meta_scale = S.meta_scale;
  float *out_row = hh < GH ? S.logits + (int64_t)(head_base + hh) * ld : nullptr;
  const bool vec_out = S.vec_out != 0;
  const int tiles_per_block = S.tiles_per_block;
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

  // Work items = (tile, pass).  The plane words of item i+1 are loaded once
  // item i is in the code table, while it is multiplied and written out.
  // Visited tile v of this block: all tiles, or (sample mode) nvtiles tiles
  // spread evenly over the ntiles real ones.
  const int nvtiles = S.nvtiles, ntiles_real = S.ntiles;
  auto real_tile = [&](int v) -> int {
    return MODE == kScanSample ? (int)((int64_t)v * ntiles_real / nvtiles) : v;
  };
  int ntiles = 0;
  while (ntiles < tiles_per_block && bw.tile0 + ntiles * bw.tile_step < nvtiles) ++ntiles;
  // item i = (tile pair i / npasses, pass): half h takes tile 2 * pair + h
  const int nitems = (ntiles + 1) / 2 * npasses;
  auto issue = [&](int item, uint32_t(&x)[32]) {
    const int ti = item / npasses, p = item - ti * npasses;
    const int tt = 2 * ti + half;
    if (tt >= ntiles) return;    // odd tile count: no tile for this half
    const int grp = kPassGroups * p + wave;
    if (grp >= ngroups) return;  // empty group: nothing to read
    const uint32_t tile_off =
        (uint32_t)real_tile(bw.tile0 + tt * bw.tile_step) * (kMTileKeys / 8);
    const uint4 dv = *reinterpret_cast<const uint4 *>(&s_desc[grp * 8]);
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t desc = __builtin_amdgcn_readfirstlane((dw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      const uint32_t c = (desc >> 3) & (kD - 1), dep = desc & 7u, top = desc >> 10;
      const uint32_t voff =
          plane_sl < dep && plane_sl >= top ? c * chan_bytes + tile_off + lane_part : kUnread;
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int32_t)voff, 0, 0);
      x[4 * i + 0] = (uint32_t)v[0];
      x[4 * i + 1] = (uint32_t)v[1];
      x[4 * i + 2] = (uint32_t)v[2];
      x[4 * i + 3] = (uint32_t)v[3];
    }
  };

  // float threshold of this lane's output row (candidate modes)
  const float row_tf = (MODE == kScanCand || MODE == kScanCandGroup) && hh < GH ? s_tf[hh] : 0.0f;
  // side stream: 4 aligned bytes per beta when rows start on 4-byte bounds
  const bool meta_words =
      META && meta && ((reinterpret_cast<uintptr_t>(S.meta) & 3) == 0) && (n & 3) == 0;

  uint32_t xn[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) xn[r] = 0;
  if (nitems > 0) issue(0, xn);
  // Ping-pong: the item sequence of half 1 runs one step behind half 0, and
  // a step (between two barriers) is either the T phase of an item (regroup,
  // next item's loads, transpose into the half's code table) or its M phase
  // (matrix cores over the code table, then the epilogue).  While one half
  // transposes, the other multiplies.
  float s[16];
  uint32_t mw[4] = {0u, 0u, 0u, 0u};  // side-stream bytes, T phase -> M phase
  const int nsteps = nitems > 0 ? 2 * nitems + 1 : 0;
  for (int k = 0; k < nsteps; ++k) {
    const int q = k - half;
    if (q >= 0 && q < 2 * nitems) {
    const int it = q >> 1;
    const int ti = it / npasses, p = it - ti * npasses;
    const int tt = 2 * ti + half;
    const bool has_tile = tt < ntiles;  // half-uniform
    const int vt = bw.tile0 + tt * bw.tile_step;
    const int64_t tile_key0 = (int64_t)real_tile(vt) * kMTileKeys;
    const bool has_group = has_tile && kPassGroups * p + wave < ngroups;
    if ((q & 1) == 0) {
    // ==== T phase
    // side-stream bytes of this tile, loaded before the next item's planes so
    // that waiting for them does not wait for those
    if (META && meta_words && has_tile && p == npasses - 1 && hh < GH) {
      mw[0] = mw[1] = mw[2] = mw[3] = 0u;
      const int64_t kb0 = tile_key0 + 256 * wave + 4 * (lane & 15);
#pragma unroll
      for (int beta = 0; beta < 4; ++beta)
        if (kb0 + 64 * beta + 4 <= n)
          mw[beta] = *reinterpret_cast<const uint32_t *>(meta + kb0 + 64 * beta);
    }
    // ---- regroup: quarter k ends with word 4*m16 + k of the 4 plane rows of
    // every slot; 32-lane halves first, then 16-lane rows.
    uint32_t(&x)[32] = xn;  // regrouped and transposed in place
    if (has_group) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto h02 = __builtin_amdgcn_permlane32_swap(x[4 * i + 0], x[4 * i + 2], false, false);
        const auto h13 = __builtin_amdgcn_permlane32_swap(x[4 * i + 1], x[4 * i + 3], false, false);
        x[4 * i + 0] = h02[0];
        x[4 * i + 2] = h02[1];
        x[4 * i + 1] = h13[0];
        x[4 * i + 3] = h13[1];
      }
    }
    if (has_group) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto r01 = __builtin_amdgcn_permlane16_swap(x[4 * i + 0], x[4 * i + 1], false, false);
        const auto r23 = __builtin_amdgcn_permlane16_swap(x[4 * i + 2], x[4 * i + 3], false, false);
        x[4 * i + 0] = r01[0];
        x[4 * i + 1] = r01[1];
        x[4 * i + 2] = r23[0];
        x[4 * i + 3] = r23[1];
      }
      // ---- transpose: x[4j+q] = bit q of slot j for keys 32w..32w+31 of the
      // tile, w = 4*m16 + quarter; afterwards x[t] = the 8 codes of key 32w+t
      transpose32_perm(x);
      const int w = 4 * m16 + quarter;
      uint32_t *dst = &codes[code_index(wave, 32 * w)];
#pragma unroll
      for (int t = 0; t < 32; ++t) dst[t] = x[t];
    }
    // the next item's words load into the same registers once these are in
    // the code table
    if (it + 1 < nitems) issue(it + 1, xn);
    } else {
    // ==== M phase
    // ---- MFMA phase: 256 keys of this wave; block b = 4*beta + e covers keys
    // 64*beta + 4*n + e (n = lane % 16)
    const int j = lane >> 4, nn = lane & 15;
    if (has_tile) {
    const int4 av = *reinterpret_cast<const int4 *>(&s_limbs[p][lane][0]);
    const v4i A = v4i{av.x, av.y, av.z, av.w};
    if (p == 0) {
#pragma unroll
      for (int b = 0; b < 16; ++b) s[b] = Ch;
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
        s[4 * beta + e] = __fmaf_rn(t, scale, s[4 * beta + e]);
      }
    }
    }  // has_tile

    // ---- epilogue: 4 consecutive keys of head hh per beta
    if (has_tile && p == npasses - 1) {
      const int64_t kb = tile_key0 + 256 * wave + 4 * nn;  // + 64*beta + e
      if (META && meta_words && hh < GH) {
#pragma unroll
        for (int b = 0; b < 16; ++b)
          s[b] = __fmaf_rn(meta_scale, (float)((mw[b >> 2] >> (8 * (b & 3))) & 0xFFu), s[b]);
      } else if (META && meta && hh < GH) {
        uint32_t mb[16];
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const int64_t key = kb + 64 * (b >> 2) + (b & 3);
          mb[b] = key < n ? meta[key] : 0u;
        }
#pragma unroll
        for (int b = 0; b < 16; ++b) s[b] = __fmaf_rn(meta_scale, (float)mb[b], s[b]);
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
            for (int b = 0; b < 16; ++b) {
              const int64_t off = 64 * (b >> 2) + (b & 3);
              if (kb + off < n) op[off] = s[b];
            }
          }
        }
      } else if constexpr (MODE == kScanSample) {
        // sampled tile vt lands at vt * 2048 of the head's sample row; keys
        // past n read as -inf
        if (hh < GH) {
          float *op = S.sample + (int64_t)(head_base + hh) * kSampleKeys +
                      (int64_t)vt * kMTileKeys + 256 * wave + 4 * nn;
#pragma unroll
          for (int beta = 0; beta < 4; ++beta) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v4[e] = kb + 64 * beta + e < n ? s[4 * beta + e] : -INFINITY;
            *reinterpret_cast<float4 *>(op + 64 * beta) = make_float4(v4[0], v4[1], v4[2], v4[3]);
          }
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
          for (int b = 0; b < 16; ++b) {
            // rows of 16 lanes are heads; row 0 receives rows 1, 2, 3 by
            // lane-row swaps (VALU, no LDS round trip)
            const uint32_t v = __float_as_uint(s[b]);
            const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            const auto p48 = __builtin_amdgcn_permlane16_swap(p32[1], p32[1], false, false);
            const float s1 = __uint_as_float(p16[1]);
            const float s2 = __uint_as_float(p32[1]);
            const float s3 = __uint_as_float(p48[1]);
            float approx = s[b], mag = fabsf(s[b]);
            if (GH > 1) { approx = __fadd_rn(approx, s1); mag = __fadd_rn(mag, fabsf(s1)); }
            if (GH > 2) { approx = __fadd_rn(approx, s2); mag = __fadd_rn(mag, fabsf(s2)); }
            if (GH > 3) { approx = __fadd_rn(approx, s3); mag = __fadd_rn(mag, fabsf(s3)); }
            const float margin = __fmaf_rn(mag, 4.76837158203125e-07f /* 2^-21 */,
                                           1.1754943508222875e-38f /* 2^-126 */);
            const bool near = hh == 0 && __fadd_rn(approx, margin) >= row_tf;
            if (__ballot(near) != 0ull) {
              double acc = (double)s[b];
              if (GH > 1) acc = __dadd_rn(acc, (double)s1);
              if (GH > 2) acc = __dadd_rn(acc, (double)s2);
              if (GH > 3) acc = __dadd_rn(acc, (double)s3);
              s[b] = (float)acc;
            } else {
              s[b] = approx;
            }
          }
          lane_rows = hh == 0;
          row = g;
        }
        if (lane_rows) {
          // s >= t as floats is to_key(s) >= T (see key_threshold); keys
          // kb + 64*beta + e are valid while 64*beta + e < lim
          const int64_t rem = n - kb;
          const int lim = rem > 256 ? 256 : (int)rem;
          uint32_t mask = 0;
#pragma unroll
          for (int b = 0; b < 16; ++b)
            mask |= (uint32_t)((64 * (b >> 2) + (b & 3) < lim) && s[b] >= row_tf) << b;
          if (mask) {
            // this block's segment of the row's candidate store
            uint32_t pos = atomicAdd(&s_segc[MODE == kScanCandGroup ? 0 : hh],
                                     (uint32_t)__popc(mask));
            uint64_t *cl = S.cand + (int64_t)row * kFusedCap + (int64_t)bw.tile0 * S.seg_cap;
            while (mask) {
              const int b = __ffs(mask) - 1;
              mask &= mask - 1;
              if (pos < (uint32_t)S.seg_cap) {
                float v = s[0];
#pragma unroll
                for (int q = 1; q < 16; ++q) v = b == q ? s[q] : v;
                cl[pos] = compose(to_key(v), kb + 64 * (b >> 2) + (b & 3));
              }
              ++pos;
            }
          }
        }
      }
    }
    }  // M phase
    }  // q in range
    __syncthreads();
  }
  if constexpr (MODE == kScanCand || MODE == kScanCandGroup) {
    // every block reports its count (above seg_cap: the segment overflowed)
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

template <int AUX>
ScanFn pick(int GH) {
  switch (GH) {
    case 1: return scan_kernel<1, AUX>;
    case 2: return scan_kernel<2, AUX>;
    case 3: return scan_kernel<3, AUX>;
    default: return scan_kernel<4, AUX>;
  }
}

template <int MODE, bool META>
ScanFn pick_mfma_mode(int GH) {
  switch (GH) {
    case 1: return scan_mfma_kernel<1, MODE, META>;
    case 2: return scan_mfma_kernel<2, MODE, META>;
    case 3: return scan_mfma_kernel<3, MODE, META>;
    default: return scan_mfma_kernel<4, MODE, META>;
  }
}

template <bool META>
ScanFn pick_mfma_meta(int GH, int mode) {
  switch (mode) {
    case kScanSample: return pick_mfma_mode<kScanSample, META>(GH);
    case kScanCand: return pick_mfma_mode<kScanCand, META>(GH);
    case kScanCandGroup: return pick_mfma_mode<kScanCandGroup, META>(GH);
    default: return pick_mfma_mode<kScanLogits, META>(GH);
  }
}

ScanFn pick_mfma(int GH, int mode, bool meta) {
  return meta ? pick_mfma_meta<true>(GH, mode) : pick_mfma_meta<false>(GH, mode);
}

// Pinned-host planes: the link is the bound, the fp32 kernel with whole-word
// lanes keeps 256-byte wave accesses.  HBM planes: the matrix-core kernel
// (the fp32 kernel above 2^25 keys per session).
ScanFn kernel_for(bool host, int GH, int mode, bool meta) {
  return host ? pick<kHostAux>(GH) : pick_mfma(GH, mode, meta);
}
int threads_for(bool host) { return host ? kScanThreads : kMThreads; }

int resident_blocks_per_cu(bool host, int GH, int mode, bool meta) {
  static int cached[2][kMaxGH + 1][4][2] = {};
  int &c = cached[host ? 1 : 0][GH][mode][meta ? 1 : 0];
  if (c == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, kernel_for(host, GH, mode, meta), threads_for(host), 0);
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
                    hipStream_t s, int32_t mode, int32_t *nseg_out, bool one_block_per_head) {
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
    if (fp32_path && sess[j].redo) {
      set_error("scan: recompute flags need the matrix-core scan");
      return FATHOM_ERR_UNSUPPORTED;
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
        resident_blocks_per_cu(fp32_path, std::min(kMaxGH, group), kernel_mode, any_meta);
    int64_t tpb_s[kSessPerLaunch];
    for (int j = 0; j < cnt; ++j) {
      const int64_t tiles = visited(sess[s0 + j].n);
      int64_t tpb = 1;
      if (one_block_per_head) tpb = std::max<int64_t>(1, tiles);
      if (total_tiles > target_blocks) tpb = std::max(tpb, (total_tiles + target_blocks - 1) / target_blocks);
      if (cand) tpb = std::max(tpb, (tiles + kMaxSeg - 1) / kMaxSeg);  // segments per row
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
      int32_t blocks = 0;
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
        o.vec_out = ((reinterpret_cast<uintptr_t>(in.logits) & 15) == 0) && (in.ld % 4 == 0);
        o.sample = in.sample;
        o.thr = in.thr;
        o.cand = in.cand;
        o.seg_cnt = in.seg_cnt;
        o.redo = in.redo;
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
      hipLaunchKernelGGL(kernel_for(fp32_path, GH, mode, any_meta), dim3(blocks),
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
