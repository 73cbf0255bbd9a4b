// salad_linear_state_noalloc: the linear-attention state of
// salad_linear_state with its split-N partial states in a file-scope device
// array instead of a caller workspace, for callers that cannot allocate
// device memory at all.
//
// The array is a fixed-size __device__ object of this code object: every
// GPU the library runs on holds its own copy from module load until the
// process ends, at its own device address.  Host code never passes the
// array's name to a kernel (in host code that name is a host-side shadow,
// not a device address): the first call on a device looks the address up
// with hipGetSymbolAddress while that device is current and keeps it, and
// every later call on that device uses the kept pointer.
//
// Calls on one GPU share that GPU's array: two calls whose kernels overlap
// on one device (different streams, or different host threads) race on it.
// Each call overwrites every partial state it reads, so nothing has to be
// cleared between calls.
#include <mutex>

#include "../../include/salad.h"
#include "common.h"
#include "kernels.h"

namespace salad {

// 36 MiB: split-N partial states of B*H*S*(d*d + d) floats; the split count
// keeps B*H*S <= 512 for B*H <= 512, which is 33.8 MB at d = 128.
constexpr size_t kNoAllocScratchBytes = size_t(36) << 20;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (looked up once per device).
hipError_t noalloc_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

}  // namespace salad
