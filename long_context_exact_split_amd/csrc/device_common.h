// Device helpers shared by the gfx950 decode kernels: lane-group reductions
// built from DPP row operations, bfloat16 widening, and small math wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15-i within a row of 16
constexpr int kDppRowHalfMirror = 0x141;// lane i <- lane 7-i within each half row

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, true));
}

// The values of lanes l and l ^ OFF (OFF in {8, 16, 32}) as (a, b), with
// lane-crossing VALU operations: a row rotation by 8 (DPP) within a row of 16,
// v_permlane16_swap across row pairs, v_permlane32_swap across wave halves.
// For OFF = 16 and 32 both lanes of a pair get the same (a, b); for OFF = 8,
// a is the lane's own value.  A commutative combination of a and b is
// therefore identical in both lanes of the pair.
//
// The swap builtins return a two-element vector; each element is copied to a
// scalar before the bit cast to float, because a bit cast applied to the
// element expression itself reads element 0 with this compiler.
constexpr int kDppRowRor8 = 0x128;  // row_ror:8

template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float &a, float &b) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane distance");
  if constexpr (OFF == 8) {
    a = x;
    b = dpp_f32<kDppRowRor8>(x);
  } else {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    uint32_t r0, r1;
    if constexpr (OFF == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      r0 = r[0];
      r1 = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      r0 = r[0];
      r1 = r[1];
    }
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
  }
}

// All-reduce (sum) over aligned groups of N lanes, N in {1, 2, 4, 8, 16, 32, 64}.
// Within a row of 16 lanes the butterfly uses DPP: after the two quad steps
// every lane holds its quad's sum, the half-row mirror pairs quad 0 with
// quad 1 (and 2 with 3), the row mirror pairs the two halves.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowMirror>(x);
  float a, b;
  if constexpr (N >= 32) {
    lane_pair<16>(x, a, b);
    x = a + b;
  }
  if constexpr (N >= 64) {
    lane_pair<32>(x, a, b);
    x = a + b;
  }
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  float a, b;
  lane_pair<16>(x, a, b);
  x = fmaxf(a, b);
  lane_pair<32>(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }



__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) x += __shfl_xor(x, off);
  return x;
}

// bfloat16 pair (little-endian: element 2e in the low half) -> two floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// e^(a-b) in base 2 with the identity record guarded: 0 when a is -inf.
__device__ __forceinline__ float rescale_factor(float a, float b) {
  return a == -INFINITY ? 0.0f : fast_exp2(a - b);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

}  // namespace attn
