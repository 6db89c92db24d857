// lora_apply_noalloc: lora_apply with its workspace taken from a fixed,
// library-owned device array instead of a caller buffer, for callers that
// cannot allocate device memory at call time (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array lives for the whole process: a file-scope device variable, one
// copy per GPU the library's code object is loaded on.  Its device address is
// looked up once per device (hipGetSymbolAddress) and only that address is
// ever handed to kernels or copies; the variable's name in host code is a
// host-side stand-in, not a device address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "lora.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (NULL on a HIP error).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // the same address on every lookup: concurrent first calls store the same value
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

lora_status_t lora_apply_noalloc(const int32_t* ids, const lora_segments_t* segs, int32_t T,
                                 const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                                 const lora_pool_t* pool, void* stream) {
  if (T < 0 || n_projs < 0 || (n_projs > 0 && !projs) || !adapters) return LORA_ERR_INVALID_ARG;
  int32_t max_d_in = 0;
  for (int i = 0; i < n_projs; ++i) max_d_in = std::max(max_d_in, projs[i].d_in);
  const size_t need = lora_workspace_size(T, adapters->num_adapters, n_projs, max_d_in);
  // 0: arguments outside the limits, which lora_apply reports precisely
  if (need > kScratchBytes) return LORA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return LORA_ERR_HIP;
  return lora_apply(ids, segs, T, projs, n_projs, adapters, pool, ws, kScratchBytes, stream);
}

}  // extern "C"
