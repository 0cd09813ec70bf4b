// attn_bwd_noalloc: the backward of attn_bwd for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  Its workspace (the per-row D and the float32 partials
// of divided passes) lives in a fixed device array of this file instead of a
// caller buffer, so the call needs no allocation from anyone.
//
// The array is a file-scope __device__ object: every device the library runs
// on holds its own copy at its own address until the process ends.  On the
// host its name is only a stand-in, so the device address is resolved once
// per device with hipGetSymbolAddress (on the first call made with that
// device current) and kept; kernels receive that address like any other
// workspace pointer.  Every call on a device shares that device's array:
// calls that overlap on one device (on different streams, or from different
// host threads without ordering) race.  Nothing in the array needs to start
// at zero: every pass writes what it later reads.
#include <hip/hip_runtime.h>

#include <atomic>

#include "attn_internal.h"

namespace attn {

constexpr size_t kScratchBytes = ATTN_BWD_NOALLOC_MAX_WORKSPACE;  // per device
static_assert(kScratchBytes % 256 == 0, "scratch is a whole number of 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// device -> address of that device's copy of `scratch` (null until resolved)
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

}  // namespace attn

using namespace attn;

extern "C" {

attn_status attn_bwd_noalloc(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                             const void* V, const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                             void* dV, void* stream) {
  const attn_status st = attn_validate(prob, mask);
  if (st != ATTN_OK) return st;
  if (attn_bwd_workspace_size(prob) > kScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (ws == nullptr) return ATTN_ERR_HIP;
  return attn_bwd(prob, mask, Q, K, V, O, lse, dO, dQ, dK, dV, ws, kScratchBytes, stream);
}

}  // extern "C"
