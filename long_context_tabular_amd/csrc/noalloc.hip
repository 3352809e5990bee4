// Library-held device scratch for sdm_icl_attn_query_noalloc: the query
// workspace (scaled query operand and the split partials) of callers that
// cannot allocate device memory.  The array lives in the code object, so each
// GPU the library runs on holds its own copy from module load until the
// process ends; its device address differs per GPU and is looked up once per
// device with that device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace sdm {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[device]) {
    // the caller made `device` current; the symbol's address is per device
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[device] = p;
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace sdm
