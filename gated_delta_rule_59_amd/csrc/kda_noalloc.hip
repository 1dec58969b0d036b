// Device scratch of kda_chunk_fwd_noalloc: a fixed array in the library's own device memory,
// for callers that cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array lives in the code object, so every GPU the library runs on holds its own copy from
// when the library's kernels are first loaded there until the process ends. In host code the
// array's name is only a stand-in: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the kernels get.
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` per device, looked up on first use

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
