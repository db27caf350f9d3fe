// Fixed device scratch for the backward entry point that allocates nothing
// (ulysses_attn_bwd_noalloc): callers under HIP graph capture, tight serving
// loops or harnesses that forbid hipMalloc cannot hand the library a
// workspace they allocated for the call.
//
// The scratch is a file-scope device array of kNoAllocScratchBytes.  Every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol, not a device address, so the address is looked up once per device
// (with that device current) through hipGetSymbolAddress and kept; kernels
// receive that pointer like any caller-provided workspace.
//
// Every call on one GPU shares that GPU's array and leaves its contents
// behind; the backward writes every statistic it later reads, so nothing
// has to start at zero.  Calls that overlap in time on one GPU (two streams,
// two host threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "ulysses.h"

namespace ulysses {

namespace {

constexpr size_t kNoAllocScratchBytes = ULYSSES_NOALLOC_SCRATCH_BYTES;   // per GPU
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU, once looked up

}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ulysses
