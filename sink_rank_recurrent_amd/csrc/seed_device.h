// Device helpers shared by the gfx950 kernels: vector loads/stores of fp32
// and bf16 data, and reductions over a 32-lane half of a wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seed {

enum RuleId { kGDN = 0, kKDA = 1, kMAMBA2 = 2 };

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Load N (2 or 4) consecutive floats.
template <int N>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  } else {
    const float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x; x[1] = t.y;
  }
}

// Load N (2 or 4) consecutive bf16 values, widened exactly to fp32.
template <int N>
__device__ __forceinline__ void load_vec(const bf16_t* __restrict__ p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_bits_to_f32(t.x & 0xffffu); x[1] = bf16_bits_to_f32(t.x >> 16);
    x[2] = bf16_bits_to_f32(t.y & 0xffffu); x[3] = bf16_bits_to_f32(t.y >> 16);
  } else {
    const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
    x[0] = bf16_bits_to_f32(t & 0xffffu); x[1] = bf16_bits_to_f32(t >> 16);
  }
}

__device__ __forceinline__ float load_scalar(const float* p) { return *p; }
__device__ __forceinline__ float load_scalar(const bf16_t* p) { return bf16_bits_to_f32(*p); }

template <int N>
__device__ __forceinline__ void store_vec(float* __restrict__ p, const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  }
}

// Sum over the 32 lanes of a half-wave (lanes 0-31 or 32-63 of a wave64),
// returned to all of them with one bit pattern.  Inside each row of 16
// lanes: DPP butterflies (xor 1, xor 2, mirror within 8, mirror within 16);
// then row_bcast:15 adds row 0's sum into row 1 (and row 2's into row 3),
// and lanes 31 and 63, which now hold the half-wave sums, are read back.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum32(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  return (__lane_id() & 32) ? hi : lo;
}

}  // namespace seed
