// Scratch memory for callers that cannot allocate (code under graph capture,
// serving loops that forbid hipMalloc): one file-scope device array that
// fathom_topk_noalloc uses in place of a caller workspace.
//
// Every GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends.  Host code never passes the array's name to a
// kernel (on the host it names a stand-in, not device memory): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  All calls on one
// GPU share its copy; calls that overlap on one GPU (two streams, two
// threads) race on it and must be ordered by the caller.
#include <mutex>

#include "fathom_internal.h"

namespace fathom {
namespace {

// The top-k workspace of FATHOM_NOALLOC_MAX_ROWS output rows (per row a
// threshold, a flag, a recompute slot, a 128-byte counter line and kCandCap
// 64-bit candidate words), padded to 256 bytes.
constexpr int64_t kSmall =
    ((3 * (int64_t)FATHOM_NOALLOC_MAX_ROWS) * 4 + 255) / 256 * 256;
constexpr int64_t kScratchBytes =
    kSmall + (int64_t)FATHOM_NOALLOC_MAX_ROWS * kCntStride * 4 +
    (int64_t)FATHOM_NOALLOC_MAX_ROWS * kCandCap * 8;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};  // each device's address of `scratch`

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

int32_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("noalloc: device %d is beyond the %d devices this library tracks", dev,
              kMaxDevices);
    return FATHOM_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "noalloc: hipGetSymbolAddress(scratch)");
    if (!p) {
      set_error("noalloc: hipGetSymbolAddress returned no address for device %d", dev);
      return FATHOM_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return FATHOM_OK;
}

}  // namespace fathom
