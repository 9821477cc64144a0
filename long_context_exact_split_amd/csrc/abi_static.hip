// attn_decode_static: attn_decode with its partial records in a device array
// of the library instead of a caller's workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array, `scratch`, is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  Host code never passes its name to a kernel (in host code the name
// is a host-side stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept; kernels get that address as their workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "abi_internal.h"
#include "attn_decode.h"

namespace {

constexpr size_t kScratchBytes = ATTN_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`.
attn_status_t scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status_t attn_decode_static(const attn_desc_t *desc, const void *q, const void *k,
                                            const void *v, float *o, float *lse, void *stream) {
  try {
    size_t need = 0;
    attn_status_t st = attn_workspace_bytes(desc, &need);
    if (st != ATTN_OK) return st;
    if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != ATTN_OK) return st;
    return attn::decode_with_workspace(desc, q, k, v, o, lse, ws, kScratchBytes, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}
