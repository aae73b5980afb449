// Library-owned scratch memory of hlq_linear_backward_noalloc: the workspace
// of the backward (quantized operands, scales, partial maxima) in a static
// device array, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library's code
// object loads on holds its own copy (HLQ_NOALLOC_SCRATCH_BYTES) until the
// process ends.  In host code its name is only a host-side stand-in, so the
// device address is resolved once per device with hipGetSymbolAddress (with
// that device current) and kept; kernels only ever receive that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/hlq.h"
#include "hlq_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[HLQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace hlq {

// Device address of the current device's scratch array (resolved on the
// first call for that device); nullptr on a runtime error.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace hlq
