// The library's one device buffer of its own: a fixed scratch array that serves as the
// workspace of paro_rotated_linear_noalloc (include/paro.h), for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy, at
// its own address, from the code object's load until the process ends. In host code its name
// stands for a host-side shadow, not a device address, so host code never passes it to a
// kernel: the first call on a device looks up that device's address with hipGetSymbolAddress
// (with the device current) and keeps it; every later use goes through the kept pointer.
//
// Every call on one GPU shares that GPU's array and it keeps the last call's contents. The
// linear's workspace needs no clearing (the transformed rows and the split partial sums are
// written in full before they are read), and calls that overlap in time on one GPU race.
#include <mutex>

#include "paro_internal.h"

namespace paro {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidValue;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace paro
