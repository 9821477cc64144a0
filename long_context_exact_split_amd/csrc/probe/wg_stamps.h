// Per-workgroup timing of a split kernel (measurement builds only: the
// product library is compiled without ATTN_WG_STAMPS and holds none of this).
//
// Each workgroup records the shader clock (s_memrealtime, a constant 100 MHz
// counter) when it starts and when its last wave is done, and the XCD and
// hardware slot it ran on, into a device array that the host reads back with
// attn_probe_wg_stamps.  The bench uses it to see how the work of one launch
// ends across the eight XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Each source that includes this has its own array (its own code object)
// and its own read-back, named by ATTN_WG_STAMPS_READBACK.
#ifndef ATTN_WG_STAMPS_READBACK
#define ATTN_WG_STAMPS_READBACK attn_probe_wg_stamps
#endif

namespace attn {
namespace probe {
namespace {

constexpr int kMaxStampedWgs = 4096;
__device__ uint64_t g_wg_stamps[kMaxStampedWgs * 4];

struct WgStamp {
  uint64_t t0;
  __device__ WgStamp() : t0(__builtin_amdgcn_s_memrealtime()) {}
  __device__ ~WgStamp() {
    __syncthreads();
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kMaxStampedWgs) {
      const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
      uint32_t xcc, hw;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
      uint64_t *s = g_wg_stamps + 4 * blockIdx.x;  // vector stores from lane 0
      s[0] = t0;
      s[1] = t1;
      s[2] = xcc;
      s[3] = hw;
    }
  }
};

}  // namespace
}  // namespace probe
}  // namespace attn

// Copies the stamps of workgroups [0, n) of the last stamped launch of this
// source's kernels to host memory: 4 values each (start clock, end clock,
// XCC id register, HW id register).  0 on success.
extern "C" __attribute__((visibility("default")))
int ATTN_WG_STAMPS_READBACK(uint64_t *host, int n) {
  if (n < 0 || n > attn::probe::kMaxStampedWgs) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(attn::probe::g_wg_stamps),
                                  sizeof(uint64_t) * 4 * (size_t)n);
}

#define ATTN_WG_STAMP() ::attn::probe::WgStamp attn_wg_stamp_
