// Device-resident scratch memory for gecko_sca_awm_forward_noalloc, the
// forward for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array below is part of the library's code object: the HIP runtime
// places one copy on every GPU the library runs on when it loads the code
// object there, and keeps it until the process ends. Its name is a host-side
// stand-in in host code, not a device address: the device address of each
// GPU's copy comes from hipGetSymbolAddress with that GPU current, is looked
// up once per device and kept, and only that address is handed to kernels.
//
// Nothing in it has to start at zero: the memory chunk pass and the scan write
// every cell of the forward's workspace that a later kernel reads, so the
// contents a previous call left behind do not matter.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gecko.h"
#include "gecko_internal.hpp"

static __device__ __align__(256) unsigned char scratch[GECKO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = GECKO_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of each GPU's copy, once looked up

}  // namespace

namespace gecko {

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[device]) {
    // the caller has made `device` current: the address returned is that GPU's copy
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[device] = p;
  }
  *ptr = g_scratch[device];
  return hipSuccess;
}

}  // namespace gecko
