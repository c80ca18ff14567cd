// Storage side of Fathom (explainer, section 核心方法, storage side): 4-bit
// per-channel min-max quantisation of K into channel-major bit planes.
//
//   pack_minmax   per-(chunk, kv head, channel) min / max partials
//   pack_range    reduce the partials -> lo, hi  (stored +0 for a -0 end)
//   pack_planes   codes -> 4 bit planes via wave64 ballots; per-block code
//                 sums S1, S2 from popcounts of the ballots (exact integers)
//   pack_sigma    sigma^2 = Var(code) * delta^2 from the exact integer sums
//
// Every value is bit-identical to the CPU definition: min/max are exact, the
// quantiser's code is floor of one IEEE fp32 subtract followed by one
// correctly rounded fp32 divide, and the variance is evaluated from exact
// int64 sums in a fixed fp64 order.
//
// Keys whose rows are 16-byte aligned take the vector kernels (16-byte loads,
// four key rows per wave instruction); other strides take the scalar ones.
//
// Per-block ranges (lo, hi kept per 2048-key block of a channel, for long
// sessions whose key ranges drift; deployment warnings item 3 and the problem
// statement): the min/max kernels run with one chunk per block and store the
// block's range directly, the planes kernels quantise each block with its own
// range, and pack_sigma_blocked pools the blocks' variances in block order.
#include <hip/hip_fp16.h>

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kMinmaxThreads = 256;
constexpr int kPlaneThreads = 256;           // 4 waves, 32 channels each
constexpr int kSubTile = 64;                 // keys per ballot (one wave)
constexpr int kLdsPitch = kD + 1;            // fp32 words per staged key row

__device__ inline float load_key(const __half *p) { return __half2float(*p); }
__device__ inline float load_key(const float *p) { return *p; }

// Partial min/max of chunk blockIdx.x for kv head blockIdx.y.
// Per-block ranges (rs > 0, chunk = one 2048-key block): the chunk's min and
// max are block blockIdx.x's range, stored (+0 for a -0 end) into
// blo/bhi[h][blockIdx.x][c] instead of part.
__device__ __forceinline__ void store_minmax(float2 *part, float *blo, float *bhi, int64_t rs,
                                             int hkv, int h, int c, float mn, float mx) {
  if (rs == 0) {
    part[((int64_t)blockIdx.x * hkv + h) * kD + c] = make_float2(mn, mx);
  } else {
    const int64_t o = ((int64_t)h * rs + blockIdx.x) * kD + c;
    blo[o] = __fadd_rn(mn, 0.0f);
    bhi[o] = __fadd_rn(mx, 0.0f);
  }
}

template <typename T>
__global__ __launch_bounds__(kMinmaxThreads) void pack_minmax_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok,
    int64_t stride_head, int64_t chunk, float2 *__restrict__ part, float *__restrict__ blo,
    float *__restrict__ bhi, int64_t rs) {
  const int h = blockIdx.y;
  const int hkv = gridDim.y;
  const int c = threadIdx.x % kD;
  const int r = threadIdx.x / kD;  // 0..1
  const int64_t i0 = (int64_t)blockIdx.x * chunk;
  const int64_t i1 = min(n, i0 + chunk);
  float mn = INFINITY, mx = -INFINITY;
  const T *base = keys + (int64_t)h * stride_head + c;
  for (int64_t i = i0 + r; i < i1; i += kMinmaxThreads / kD) {
    float x = load_key(base + i * stride_tok);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  __shared__ float2 red[kMinmaxThreads];
  red[threadIdx.x] = make_float2(mn, mx);
  __syncthreads();
  if (r == 0) {
    float2 o = red[threadIdx.x + kD];
    mn = fminf(mn, o.x);
    mx = fmaxf(mx, o.y);
    store_minmax(part, blo, bhi, rs, hkv, h, c, mn, mx);
  }
}

// One block per kv head: 8 threads per channel split the partials, then a
// reduction in LDS (min / max do not depend on the order).
constexpr int kReduceThreads = 1024;
constexpr int kReduceSlices = kReduceThreads / kD;

__global__ __launch_bounds__(kReduceThreads) void pack_range_kernel(
    const float2 *__restrict__ part, int32_t nparts, int32_t hkv,
    float *__restrict__ lo, float *__restrict__ hi) {
  __shared__ float2 red[kReduceSlices][kD];
  const int h = blockIdx.x, c = threadIdx.x % kD, sl = threadIdx.x / kD;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll 8
  for (int p = sl; p < nparts; p += kReduceSlices) {
    float2 v = part[((int64_t)p * hkv + h) * kD + c];
    mn = fminf(mn, v.x);
    mx = fmaxf(mx, v.y);
  }
  red[sl][c] = make_float2(mn, mx);
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int q = 1; q < kReduceSlices; ++q) {
      mn = fminf(mn, red[q][c].x);
      mx = fmaxf(mx, red[q][c].y);
    }
    // -0 and +0 are one key value: the stored ends are +0.
    lo[h * kD + c] = __fadd_rn(mn, 0.0f);
    hi[h * kD + c] = __fadd_rn(mx, 0.0f);
  }
}

// Range of channel c of kv head h for 2048-key block b: lo/hi are [hkv][d]
// (rs == 0) or [hkv][rs][d] per block.
__device__ __forceinline__ float range_at(const float *a, int h, int c, int64_t rs, int64_t b) {
  return rs == 0 ? a[h * kD + c] : a[((int64_t)h * rs + b) * kD + c];
}

__device__ inline int quantise(float x, float lo, float delta) {
  if (delta == 0.0f) return 0;
  float y = __fdiv_rn(__fsub_rn(x, lo), delta);
  float f = floorf(y);
  return f > 15.0f ? 15 : (int)f;
}

// One block = 2048 keys (one 64-word block of every plane row) of kv head
// blockIdx.y.  Keys are staged 64 at a time through LDS (coalesced rows),
// then each wave turns one channel column into 4 ballots (64 keys = two
// plane words per plane) for its 32 channels.
template <typename T>
__global__ __launch_bounds__(kPlaneThreads) void pack_planes_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok,
    int64_t stride_head, int64_t W, const float *__restrict__ lo,
    const float *__restrict__ hi, int64_t rs, uint32_t *__restrict__ planes,
    int2 *__restrict__ sums) {
  __shared__ float tile[kSubTile * kLdsPitch];
  const int h = blockIdx.y;
  const int hkv = gridDim.y;
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t key0 = (int64_t)blockIdx.x * kBlockKeys;

  // lane cc of this wave keeps channel (wave*32 + cc)'s range and sums
  const int my_c = wave * 32 + (lane & 31);
  const float my_lo = range_at(lo, h, my_c, rs, blockIdx.x);
  const float my_delta =
      __fmul_rn(__fsub_rn(range_at(hi, h, my_c, rs, blockIdx.x), my_lo), 0.0625f);
  int my_s1 = 0, my_s2 = 0;

  for (int sub = 0; sub < kBlockKeys / kSubTile; ++sub) {
    const int64_t kb = key0 + sub * kSubTile;
    __syncthreads();
    for (int e = threadIdx.x; e < kSubTile * kD; e += kPlaneThreads) {
      const int t = e / kD, c = e % kD;
      const int64_t i = kb + t;
      tile[t * kLdsPitch + c] =
          i < n ? load_key(keys + i * stride_tok + (int64_t)h * stride_head + c)
                : 0.0f;
    }
    __syncthreads();
    const bool valid = kb + lane < n;
    const int64_t w0 = kb / 32;
#pragma unroll 4
    for (int cc = 0; cc < 32; ++cc) {
      const int c = wave * 32 + cc;
      const float clo = __shfl(my_lo, cc);
      const float cdelta = __shfl(my_delta, cc);
      const int code = valid ? quantise(tile[lane * kLdsPitch + c], clo, cdelta) : 0;
      const uint64_t m0 = __ballot(code & 1);
      const uint64_t m1 = __ballot(code & 2);
      const uint64_t m2 = __ballot(code & 4);
      const uint64_t m3 = __ballot(code & 8);
      // lanes 0..7 store slot s = lane/2 (bit 3 - s), word half lane%2
      if (lane < 8) {
        const int s = lane >> 1;
        const uint64_t m = s == 0 ? m3 : s == 1 ? m2 : s == 2 ? m1 : m0;
        const uint32_t word = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
        planes[(((int64_t)h * kD + c) * kPlanes + s) * W + w0 + (lane & 1)] = word;
      }
      // S1 = sum code, S2 = sum code^2 from popcounts of the bit planes
      const int p0 = __popcll(m0), p1 = __popcll(m1), p2 = __popcll(m2),
                p3 = __popcll(m3);
      const int s1 = p0 + 2 * p1 + 4 * p2 + 8 * p3;
      const int s2 = p0 + 4 * p1 + 16 * p2 + 64 * p3 +
                     2 * (2 * __popcll(m0 & m1) + 4 * __popcll(m0 & m2) +
                          8 * __popcll(m0 & m3) + 8 * __popcll(m1 & m2) +
                          16 * __popcll(m1 & m3) + 32 * __popcll(m2 & m3));
      if ((lane & 31) == cc) {
        my_s1 += s1;
        my_s2 += s2;
      }
    }
  }
  if (lane < 32)
    sums[((int64_t)blockIdx.x * hkv + h) * kD + my_c] = make_int2(my_s1, my_s2);
}

// ---- vector kernels (16-byte aligned key rows) -------------------------------
// Thread t of a 256-thread block owns channels 8j..8j+7 (j = t % 16) of key
// row t / 16 of each 16-row step: a wave instruction reads 4 whole rows.
constexpr int kVecThreads = 256;
constexpr int kVecRows = kVecThreads / 16;

// The 8 channels of one key row (16 bytes of fp16 or 32 of fp32).
template <typename T>
__device__ __forceinline__ void load_row8(const T *p, uint4 (&v)[2]);
template <>
__device__ __forceinline__ void load_row8<__half>(const __half *p, uint4 (&v)[2]) {
  v[0] = *reinterpret_cast<const uint4 *>(p);
  v[1] = make_uint4(0, 0, 0, 0);
}
template <>
__device__ __forceinline__ void load_row8<float>(const float *p, uint4 (&v)[2]) {
  v[0] = *reinterpret_cast<const uint4 *>(p);
  v[1] = *reinterpret_cast<const uint4 *>(p + 4);
}
template <typename T>
__device__ __forceinline__ void unpack_row8(const uint4 (&v)[2], float (&x)[8]);
template <>
__device__ __forceinline__ void unpack_row8<__half>(const uint4 (&v)[2], float (&x)[8]) {
  const uint32_t w[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
    x[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
  }
}
template <>
__device__ __forceinline__ void unpack_row8<float>(const uint4 (&v)[2], float (&x)[8]) {
  x[0] = __uint_as_float(v[0].x);
  x[1] = __uint_as_float(v[0].y);
  x[2] = __uint_as_float(v[0].z);
  x[3] = __uint_as_float(v[0].w);
  x[4] = __uint_as_float(v[1].x);
  x[5] = __uint_as_float(v[1].y);
  x[6] = __uint_as_float(v[1].z);
  x[7] = __uint_as_float(v[1].w);
}

template <typename T>
__global__ __launch_bounds__(kVecThreads) void pack_minmax_vec_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok, int64_t stride_head,
    int64_t chunk, float2 *__restrict__ part, float *__restrict__ blo, float *__restrict__ bhi,
    int64_t rs) {
  __shared__ float s_mn[kVecRows][kD + 1], s_mx[kVecRows][kD + 1];
  const int h = blockIdx.y, hkv = gridDim.y;
  const int r = threadIdx.x >> 4, j = threadIdx.x & 15;
  const int64_t i0 = (int64_t)blockIdx.x * chunk;
  const int64_t i1 = min(n, i0 + chunk);
  const T *base = keys + (int64_t)h * stride_head + 8 * j;
  float mn[8], mx[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    mn[c] = INFINITY;
    mx[c] = -INFINITY;
  }
  int64_t i = i0 + r;
  // four rows in flight per thread
  for (; i + 3 * kVecRows < i1; i += 4 * kVecRows) {
    uint4 v[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_row8<T>(base + (i + u * kVecRows) * stride_tok, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x[8];
      unpack_row8<T>(v[u], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        mn[c] = fminf(mn[c], x[c]);
        mx[c] = fmaxf(mx[c], x[c]);
      }
    }
  }
  for (; i < i1; i += kVecRows) {
    uint4 v[2];
    load_row8<T>(base + i * stride_tok, v);
    float x[8];
    unpack_row8<T>(v, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      mn[c] = fminf(mn[c], x[c]);
      mx[c] = fmaxf(mx[c], x[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s_mn[r][8 * j + c] = mn[c];
    s_mx[r][8 * j + c] = mx[c];
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    float a = INFINITY, b = -INFINITY;
#pragma unroll
    for (int q = 0; q < kVecRows; ++q) {
      a = fminf(a, s_mn[q][c]);
      b = fmaxf(b, s_mx[q][c]);
    }
    store_minmax(part, blo, bhi, rs, hkv, h, c, a, b);
  }
}

// Code of y = fl(x - lo) >= 0 as the exact definition floor(RN(y / delta))
// (clamped to 15), without the divide in almost every case.  q = RN(y * r)
// with r = RN(1/delta) differs from y / delta by at most 2 * 2^-24 * 16 and
// RN(y / delta) from y / delta by at most 2^-24 * 16, so whenever q is at
// least 2^-14 away from every integer both have the same floor; otherwise
// (and for delta = 0, or a reciprocal out of range, where q is 0, inf or NaN)
// the correctly rounded divide decides.  Returns the code, or -1 when the
// divide must decide.
__device__ __forceinline__ int quantise_fast(float y, float r) {
  const float q = __fmul_rn(y, r);
  const float f = __builtin_amdgcn_fractf(q);
  const bool safe = fabsf(__fsub_rn(f, 0.5f)) < 0.5f - 0x1p-14f;  // false for NaN
  return safe ? (int)fminf(q, 15.5f) : -1;
}

// Stage S of a 32x32 bit transpose: swap the off-diagonal SxS blocks of
// every 2Sx2S block.
template <int S, uint32_t M>
__device__ __forceinline__ void bit_stage(uint32_t (&x)[32]) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if ((r & S) == 0) {
      const uint32_t a = x[r], b = x[r + S];
      x[r] = (a & M) | ((b << S) & ~M);
      x[r + S] = ((a >> S) & M) | (b & ~M);
    }
  }
}

// 32x32 bit transpose: on entry x[t] bit b = element (t, b); on exit x[b]
// bit t = element (t, b).  Byte permutes for the 16- and 8-bit stages,
// shift/select for the rest.
__device__ __forceinline__ void bit_transpose32(uint32_t (&x)[32]) {
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
  bit_stage<4, 0x0F0F0F0Fu>(x);
  bit_stage<2, 0x33333333u>(x);
  bit_stage<1, 0x55555555u>(x);
}

// One block = (2048-key tile, quarter Q of the channels, kv head); the blocks
// of one tile's quarters run together on one XCD, so that together they read
// whole key rows through one L2.
//  * staging: thread t takes channels 32Q + 8j .. +7 (j = t % 4) of key rows
//    t / 4, t / 4 + 64, ... (16-byte loads: a wave instruction reads the
//    quarter of 16 rows; the next batch of rows is in flight while the
//    current one is quantised) and stores each row's 8 codes as one dword of
//    nibbles in LDS;
//  * planes: wave G takes channels 32Q + 8G .. +7 and lane w the 32 keys of
//    plane word w of the tile: it reads their 32 code dwords and
//    bit-transposes them, so that word 4ci + p is bit p of channel
//    32Q + 8G + ci's codes, i.e. one plane word; a store instruction then
//    writes a whole 256-byte row segment.  S1 and S2 of the 8 channels follow
//    from popcounts of the plane words (exact integers), summed over the wave.
template <typename T>
__global__ __launch_bounds__(kVecThreads) void pack_planes_vec_kernel(
    const T *__restrict__ keys, int64_t n, int64_t stride_tok, int64_t stride_head,
    int64_t W, int32_t hkv, const float *__restrict__ lo, const float *__restrict__ hi,
    int64_t rs, uint32_t *__restrict__ planes, int2 *__restrict__ sums) {
  constexpr int kGroups = 4;                      // 8-channel groups per quarter
  constexpr int kRowsPerStep = kVecThreads / kGroups;  // 64
  constexpr int kSteps = kBlockKeys / kRowsPerStep;    // 32
  constexpr int kBatch = sizeof(T) == 2 ? 8 : 4;       // rows per lane in flight
  constexpr int kBatches = kSteps / kBatch;
  // LDS dword of (key, group): 4 per key, each 32-key run shifted by one
  // (one to one; staging stores and transpose reads meet at most two lanes
  // per bank)
  __shared__ uint32_t s_codes[kBlockKeys * kGroups + kBlockKeys / 32];
  auto cidx = [](int key, int grp) { return key * kGroups + grp + (key >> 5); };
  // Block index -> (tile, kv head) pair and quarter: the four quarters of a
  // pair are 8 indices apart, which the dispatcher's round robin over the 8
  // XCDs places on one XCD back to back, so the quarter rows of a key (parts
  // of the same cache lines) meet in one L2 instead of being fetched by two.
  const int bx = blockIdx.x;
  const int pair = (bx >> 5) * 8 + (bx & 7);
  const int Q = (bx >> 3) & 3;
  if (pair >= (int)(W / 64) * hkv) return;  // padding of the last group of 8 pairs
  const int h = pair % hkv, tile = pair / hkv;
  const int tid = threadIdx.x;
  const int jr = tid >> 2, j = tid & 3;     // staging: row offset, channel group
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t key0 = (int64_t)tile * kBlockKeys;
  const int cbase = 32 * Q + 8 * j;         // this thread's staging channels
  const T *base = keys + (int64_t)h * stride_head + cbase;

  float clo[8], cdel[8], crec[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float l = range_at(lo, h, cbase + c, rs, tile);
    clo[c] = l;
    cdel[c] = __fmul_rn(__fsub_rn(range_at(hi, h, cbase + c, rs, tile), l), 0.0625f);
    crec[c] = __fdiv_rn(1.0f, cdel[c]);
  }

  auto load_batch = [&](int bt, uint4 (&v)[kBatch][2]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int64_t i = key0 + (int64_t)(bt * kBatch + u) * kRowsPerStep + jr;
      i = i < n ? i : n - 1;  // rows past n: any valid row, codes cleared below
      load_row8<T>(base + i * stride_tok, v[u]);
    }
  };
  uint4 vn[kBatch][2];
  load_batch(0, vn);
#pragma unroll 1
  for (int bt = 0; bt < kBatches; ++bt) {
    uint4 v[kBatch][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      v[u][0] = vn[u][0];
      v[u][1] = vn[u][1];
    }
    if (bt + 1 < kBatches) load_batch(bt + 1, vn);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      float x[8];
      unpack_row8<T>(v[u], x);
      int code[8];
      bool exact = false;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        code[c] = quantise_fast(__fsub_rn(x[c], clo[c]), crec[c]);
        exact |= code[c] < 0;
      }
      if (exact) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (code[c] < 0) code[c] = quantise(x[c], clo[c], cdel[c]);
      }
      const int key = (bt * kBatch + u) * kRowsPerStep + jr;
      uint32_t w = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) w |= (uint32_t)code[c] << (4 * c);
      s_codes[cidx(key, j)] = key0 + key < n ? w : 0u;
    }
  }
  __syncthreads();

  // ---- planes and code sums: wave = channel group, lane = plane word
  uint32_t x[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) x[t] = s_codes[cidx(32 * lane + t, wave)];
  bit_transpose32(x);
  // this kv head's planes (at most 2 GiB: the launcher checks); lane offset
  // of the group's first row plus the wave-uniform offset of row 4ci + s
  const uint32_t row_bytes = (uint32_t)W * 4u;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      planes + (int64_t)h * kD * kPlanes * W, (short)0, (int32_t)(row_bytes * kD * kPlanes),
      0x00020000);
  const int c0 = 32 * Q + 8 * wave;
  const uint32_t voff = (uint32_t)c0 * kPlanes * row_bytes + (uint32_t)(tile * 64 + lane) * 4u;
  int s1[8], s2[8];
#pragma unroll
  for (int ci = 0; ci < 8; ++ci) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      __builtin_amdgcn_raw_buffer_store_b32(x[4 * ci + p], prs, (int32_t)voff,
                                            (int32_t)((4 * ci + 3 - p) * row_bytes), 0);
    const uint32_t b0 = x[4 * ci], b1 = x[4 * ci + 1], b2 = x[4 * ci + 2], b3 = x[4 * ci + 3];
    const int p0 = __popc(b0), p1 = __popc(b1), p2 = __popc(b2), p3 = __popc(b3);
    s1[ci] = p0 + 2 * p1 + 4 * p2 + 8 * p3;
    s2[ci] = p0 + 4 * p1 + 16 * p2 + 64 * p3 +
             2 * (2 * __popc(b0 & b1) + 4 * __popc(b0 & b2) + 8 * __popc(b0 & b3) +
                  8 * __popc(b1 & b2) + 16 * __popc(b1 & b3) + 32 * __popc(b2 & b3));
  }
  // sums over the wave's 64 lanes (integers: the order does not matter)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int ci = 0; ci < 8; ++ci) {
      s1[ci] += __shfl_xor(s1[ci], off);
      s2[ci] += __shfl_xor(s2[ci], off);
    }
  if (lane < 8) {
    int a = s1[0], b = s2[0];
#pragma unroll
    for (int ci = 1; ci < 8; ++ci) {
      a = lane == ci ? s1[ci] : a;
      b = lane == ci ? s2[ci] : b;
    }
    sums[((int64_t)tile * hkv + h) * kD + c0 + lane] = make_int2(a, b);
  }
}

// One block per kv head: 8 threads per channel split the blocks' code sums
// (exact integers, so the order does not matter), then sigma^2 in a fixed
// fp64 order.
__global__ __launch_bounds__(kReduceThreads) void pack_sigma_kernel(
    const int2 *__restrict__ sums, int32_t nblocks, int32_t hkv, int64_t n,
    const float *__restrict__ lo, const float *__restrict__ hi,
    float *__restrict__ sigma2) {
  __shared__ longlong2 red[kReduceSlices][kD];
  const int h = blockIdx.x, c = threadIdx.x % kD, sl = threadIdx.x / kD;
  int64_t s1 = 0, s2 = 0;
#pragma unroll 8
  for (int b = sl; b < nblocks; b += kReduceSlices) {
    int2 v = sums[((int64_t)b * hkv + h) * kD + c];
    s1 += v.x;
    s2 += v.y;
  }
  red[sl][c] = make_longlong2(s1, s2);
  __syncthreads();
  if (sl != 0) return;
#pragma unroll
  for (int q = 1; q < kReduceSlices; ++q) {
    s1 += red[q][c].x;
    s2 += red[q][c].y;
  }
  const float l = lo[h * kD + c];
  const float delta = __fmul_rn(__fsub_rn(hi[h * kD + c], l), 0.0625f);
  const int64_t num = n * s2 - s1 * s1;
  const double var_code = __ddiv_rn((double)num, __dmul_rn((double)n, (double)n));
  const double dd = __dmul_rn((double)delta, (double)delta);
  sigma2[h * kD + c] = (float)__dmul_rn(var_code, dd);
}

// Per-block ranges: sigma2 = fp32(sum_b fp64(var_b * (n_b / n))), var_b =
// Var(code) * delta_b^2 of block b from its exact integer code sums (the
// expression of pack_sigma for one block).  One block of threads per kv head:
// first every (block, channel) term in parallel, written over its own code
// sums; then one thread per channel adds its terms in block order.  Each step
// is one correctly rounded fp64 operation, so the result is the CPU
// definition's bit for bit.
__global__ __launch_bounds__(kReduceThreads) void pack_sigma_blocked_kernel(
    int2 *__restrict__ sums, int32_t nblocks, int32_t hkv, int64_t n,
    const float *__restrict__ lo, const float *__restrict__ hi, int64_t rs,
    float *__restrict__ sigma2) {
  const int h = blockIdx.x, c = threadIdx.x % kD;
  double *terms = reinterpret_cast<double *>(sums);  // same 8 bytes per (block, channel)
  for (int32_t b = threadIdx.x / kD; b < nblocks; b += kReduceSlices) {
    const int64_t e = ((int64_t)b * hkv + h) * kD + c;
    const int2 v = sums[e];
    const int64_t nb = min((int64_t)kBlockKeys, n - (int64_t)b * kBlockKeys);
    const int64_t r = ((int64_t)h * rs + b) * kD + c;
    const float delta = __fmul_rn(__fsub_rn(hi[r], lo[r]), 0.0625f);
    const int64_t num = nb * (int64_t)v.y - (int64_t)v.x * (int64_t)v.x;
    const double var_code = __ddiv_rn((double)num, __dmul_rn((double)nb, (double)nb));
    const double var = __dmul_rn(var_code, __dmul_rn((double)delta, (double)delta));
    terms[e] = __dmul_rn(var, __ddiv_rn((double)nb, (double)n));
  }
  __syncthreads();
  if (threadIdx.x >= kD) return;
  double acc = 0.0;
  for (int32_t b = 0; b < nblocks; ++b) acc = __dadd_rn(acc, terms[((int64_t)b * hkv + h) * kD + c]);
  sigma2[h * kD + c] = (float)acc;
}

struct PackLayout {
  int64_t chunk;
  int32_t nparts;
  int32_t nblocks;
  int64_t part_bytes;
  int64_t sums_bytes;
};

PackLayout pack_layout(int64_t n, int32_t hkv) {
  PackLayout L;
  // enough min/max blocks to fill the chip, each at least 256 keys
  int64_t parts = (2048 + hkv - 1) / hkv;
  parts = std::min<int64_t>(parts, (n + 255) / 256);
  parts = std::max<int64_t>(parts, 1);
  L.chunk = (n + parts - 1) / parts;
  L.nparts = (int32_t)((n + L.chunk - 1) / L.chunk);
  L.nblocks = (int32_t)(plane_words(n) / 64);
  L.part_bytes = ((int64_t)L.nparts * hkv * kD * sizeof(float2) + 255) / 256 * 256;
  L.sums_bytes = (int64_t)L.nblocks * hkv * kD * sizeof(int2);
  return L;
}

// Workspace of the per-block pack: the blocks' code sums only (the min/max
// kernels store the ranges themselves).
int64_t pack_blocked_ws(int64_t n, int32_t hkv) {
  return plane_words(n) / 64 * hkv * kD * (int64_t)sizeof(int2);
}

template <typename T>
int32_t launch_pack_t(const T *keys, int64_t n, int32_t hkv, int64_t stride_tok,
                      int64_t stride_head, uint32_t *planes, float *lo,
                      float *hi, int64_t rs, float *sigma2, void *ws, hipStream_t s) {
  PackLayout L = pack_layout(n, hkv);
  if (rs > 0) {  // one min/max chunk per 2048-key block, no partials
    L.chunk = kBlockKeys;
    L.nparts = L.nblocks;
    L.part_bytes = 0;
  }
  float2 *part = reinterpret_cast<float2 *>(ws);
  int2 *sums = reinterpret_cast<int2 *>(static_cast<char *>(ws) + L.part_bytes);
  const int64_t W = plane_words(n);
  // 8 channels of a row are 16 (fp16) or 32 (fp32) bytes: vector loads need
  // 16-byte aligned rows
  constexpr int64_t kAlign = 16 / sizeof(T);
  // (and the planes kernel addresses one kv head's planes with 32-bit offsets)
  const bool vec = (reinterpret_cast<uintptr_t>(keys) % 16) == 0 && stride_tok % kAlign == 0 &&
                   stride_head % kAlign == 0 && W * 4 * kPlanes * kD <= INT32_MAX;
  if (vec)
    hipLaunchKernelGGL(pack_minmax_vec_kernel<T>, dim3(L.nparts, hkv), dim3(kVecThreads), 0, s,
                       keys, n, stride_tok, stride_head, L.chunk, part, lo, hi, rs);
  else
    hipLaunchKernelGGL(pack_minmax_kernel<T>, dim3(L.nparts, hkv), dim3(kMinmaxThreads),
                       0, s, keys, n, stride_tok, stride_head, L.chunk, part, lo, hi, rs);
  if (rs == 0)
    hipLaunchKernelGGL(pack_range_kernel, dim3(hkv), dim3(kReduceThreads), 0, s, part,
                       L.nparts, hkv, lo, hi);
  if (vec)
    hipLaunchKernelGGL(pack_planes_vec_kernel<T>,
                       dim3((unsigned)(((int64_t)L.nblocks * hkv + 7) / 8 * 32)), dim3(kVecThreads),
                       0, s, keys, n, stride_tok, stride_head, W, hkv, lo, hi, rs, planes, sums);
  else
    hipLaunchKernelGGL(pack_planes_kernel<T>, dim3(L.nblocks, hkv), dim3(kPlaneThreads),
                       0, s, keys, n, stride_tok, stride_head, W, lo, hi, rs, planes, sums);
  if (rs == 0)
    hipLaunchKernelGGL(pack_sigma_kernel, dim3(hkv), dim3(kReduceThreads), 0, s, sums,
                       L.nblocks, hkv, n, lo, hi, sigma2);
  else
    hipLaunchKernelGGL(pack_sigma_blocked_kernel, dim3(hkv), dim3(kReduceThreads), 0, s, sums,
                       L.nblocks, hkv, n, lo, hi, rs, sigma2);
  return hip_fail(hipGetLastError(), "pack launch");
}

}  // namespace

int64_t pack_workspace_bytes(int64_t n, int32_t hkv) {
  const PackLayout L = pack_layout(n, hkv);
  return L.part_bytes + L.sums_bytes;
}

int64_t pack_blocked_workspace_bytes(int64_t n, int32_t hkv) { return pack_blocked_ws(n, hkv); }

int32_t launch_pack(const void *keys, int32_t dtype, int64_t n, int32_t hkv,
                    int64_t stride_tok, int64_t stride_head, uint32_t *planes,
                    float *lo, float *hi, int64_t rs, float *sigma2, void *ws, hipStream_t s) {
  if (dtype == FATHOM_F16)
    return launch_pack_t(static_cast<const __half *>(keys), n, hkv, stride_tok,
                         stride_head, planes, lo, hi, rs, sigma2, ws, s);
  return launch_pack_t(static_cast<const float *>(keys), n, hkv, stride_tok,
                       stride_head, planes, lo, hi, rs, sigma2, ws, s);
}

}  // namespace fathom
