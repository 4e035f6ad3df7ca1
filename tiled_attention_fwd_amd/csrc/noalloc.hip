// Library-owned scratch memory for callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The paged-cache call splits long key ranges into parts whose partial
// outputs and log-sum-exps live in scratch memory until a merge launch
// combines them.  attn_fwd_paged takes that memory from the caller;
// attn_fwd_paged_noalloc uses this file-scope device array instead.  Each GPU
// the library runs on holds its own copy of the array (at its own address)
// until the process ends.  In host code the array's name is only a host-side
// stand-in, so the device address is looked up once per device with
// hipGetSymbolAddress and every later use goes through that pointer.

#include "attn_internal.h"
#include "../../include/attn_fwd.h"

#include <mutex>

namespace attnfwd {

// Every default plan of the paged call fits: parts are added only while the
// launch has fewer than 256 workgroups, so a plan holds at most 510
// (sequence, KV head, row block, part) slots of 32 rows x (head_dim + 1)
// floats, 16.8 MB at head_dim 256 (8.4 MB at 128); the planner checks this
// bound at compile time.
constexpr int64_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    // the current device is `dev`: its copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace attnfwd
