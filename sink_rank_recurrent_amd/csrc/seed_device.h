// Device helpers shared by the gfx950 kernels: vector loads/stores of fp32
// and bf16 data, reductions over a 32-lane half of a wave64, and the 16-bit
// storage formats of the factors (widening, rounding, and the Philox
// counter-based generator that stochastic rounding draws from).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "seed_launch.h"

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

// Non-temporal forms of load_vec / store_vec for data that is streamed once
// per launch (factor columns, dense states): the same 8- or 16-byte
// accesses, marked so the caches do not keep them for reuse that never
// comes (a layer's state is not touched again before every other layer's
// has streamed through).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void load_vec_nt(const float* __restrict__ p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  } else {
    const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    x[0] = t.x; x[1] = t.y;
  }
}
template <int N>
__device__ __forceinline__ void store_vec_nt(float* __restrict__ p, const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
  } else {
    __builtin_nontemporal_store(f32x2{x[0], x[1]}, reinterpret_cast<f32x2*>(p));
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

// ---------------------------------------------------------------------------
// 16-bit factor storage (StoreFmt in seed_launch.h).  kStoreF32 is the
// all-fp32 layout; with kStoreBF16 or kStoreF16 the R columns a compression
// writes are held as 16-bit patterns and every other column in fp32.

// (Instantiated with kStoreF32 only in branches that the fp32 layout never
// takes; it reads the pattern as bf16 there.)
template <int FMT>
__host__ __device__ __forceinline__ float widen16(uint32_t h16) {
  if constexpr (FMT == kStoreF16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
  } else {
    return __builtin_bit_cast(float, h16 << 16);
  }
}

// N (2 or 4) consecutive 16-bit patterns, widened exactly.
template <int FMT, int N>
__device__ __forceinline__ void load_vec16(const uint16_t* __restrict__ p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    x[0] = widen16<FMT>(t.x & 0xffffu); x[1] = widen16<FMT>(t.x >> 16);
    x[2] = widen16<FMT>(t.y & 0xffffu); x[3] = widen16<FMT>(t.y >> 16);
  } else {
    const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
    x[0] = widen16<FMT>(t & 0xffffu); x[1] = widen16<FMT>(t >> 16);
  }
}

// load_vec16 with a non-temporal access (see load_vec_nt).
template <int FMT, int N>
__device__ __forceinline__ void load_vec16_nt(const uint16_t* __restrict__ p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    x[0] = widen16<FMT>(t.x & 0xffffu); x[1] = widen16<FMT>(t.x >> 16);
    x[2] = widen16<FMT>(t.y & 0xffffu); x[3] = widen16<FMT>(t.y >> 16);
  } else {
    const uint32_t t = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    x[0] = widen16<FMT>(t & 0xffffu); x[1] = widen16<FMT>(t >> 16);
  }
}

// Round to nearest, ties to the even pattern.  bf16: the carry of
// 0x7fff + (bit 16) into the kept half does exactly that, overflow included;
// NaN stays a (quiet) NaN.  fp16: the hardware conversion, which rounds to
// nearest-even in the default mode and overflows to infinity.
template <int FMT>
__host__ __device__ __forceinline__ uint32_t round_nearest16(float x) {
  if constexpr (FMT == kStoreBF16) {
    uint32_t b = __builtin_bit_cast(uint32_t, x);
    if ((b & 0x7f800000u) == 0x7f800000u) return (b >> 16) | ((b & 0x7fffffu) ? 0x40u : 0u);
    b += 0x7fffu + ((b >> 16) & 1u);
    return b >> 16;
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

// Store N (2 or 4) floats as consecutive 16-bit patterns, rounded to nearest.
template <int FMT, int N>
__device__ __forceinline__ void store_vec16_nearest(uint16_t* __restrict__ p, const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "vector width");
  if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) =
        make_uint2(round_nearest16<FMT>(x[0]) | (round_nearest16<FMT>(x[1]) << 16),
                   round_nearest16<FMT>(x[2]) | (round_nearest16<FMT>(x[3]) << 16));
  } else {
    *reinterpret_cast<uint32_t*>(p) = round_nearest16<FMT>(x[0]) | (round_nearest16<FMT>(x[1]) << 16);
  }
}

// Stochastic rounding: with lo <= |x| < hi the adjacent magnitudes of the
// format, the magnitude goes to hi iff (|x| - lo)/(hi - lo) > u, where
// u = (w >> 8) 2^-24.  In integers: the dropped low bits D of the fp32
// pattern (2^m (|x| - lo)/(hi - lo) = D) against u: up iff D 2^(24-m) > u.
// Magnitudes from 2^16 up become infinity in fp16.
template <int FMT>
__host__ __device__ __forceinline__ uint32_t round_stochastic16(float x, uint32_t w) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const uint32_t u = w >> 8;
  if constexpr (FMT == kStoreBF16) {
    if ((b & 0x7f800000u) == 0x7f800000u) return (b >> 16) | ((b & 0x7fffffu) ? 0x40u : 0u);
    return (b >> 16) + (((b & 0xffffu) << 8) > u ? 1u : 0u);
  } else {
    const uint32_t sign = (b >> 16) & 0x8000u;
    const uint32_t m = b & 0x7fffffffu;
    if (m >= 0x47800000u) return sign | (m > 0x7f800000u ? 0x7e00u : 0x7c00u);
    const int e = (int)(m >> 23) - 127;
    if (e >= -14) {
      // fp16 normal range: 13 dropped bits
      const uint32_t h = ((uint32_t)(e + 15) << 10) | ((m >> 13) & 0x3ffu);
      return sign | (h + (((m & 0x1fffu) << 11) > u ? 1u : 0u));
    }
    // fp16 subnormal range, in units of 2^-24: |x| = M 2^-s with the 24-bit
    // significand M; lo = M >> s and D = M mod 2^s, up iff D 2^24 > u 2^s
    const bool sub32 = (m >> 23) == 0;
    const uint32_t M = sub32 ? m : ((m & 0x7fffffu) | 0x800000u);
    const int s = sub32 ? 125 : -(e + 1);
    uint32_t lo, up;
    if (s < 24) {
      lo = M >> s;
      up = ((M & ((1u << s) - 1u)) << (24 - s)) > u ? 1u : 0u;
    } else {
      lo = 0u;
      const int t = s - 24;
      up = (t >= 24) ? ((u == 0u && M != 0u) ? 1u : 0u)
                     : (((uint64_t)u << t) < (uint64_t)M ? 1u : 0u);
    }
    return sign | (lo + up);
  }
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011): ten rounds on a 4 x 32-bit counter, each two
// 32 x 32 -> 64-bit products mixed with the key, the key advanced by the
// Weyl increments between rounds.  The counter is replaced by the output.
__host__ __device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
  }
}

// Four consecutive elements f0 .. f0 + 3 (f0 a multiple of 4) of a unit's
// rank-R factor block -- U column c row i at f = c d_k + i, then V column c
// row i at f = R d_k + c d_v + i -- rounded and packed into two words.
// Stochastic rounding takes word f mod 4 of Philox(counter = (f0 / 4, unit,
// epoch, 0), key = (seed low, seed high)).
template <int FMT>
__device__ __forceinline__ uint2 round_pack4(const float (&x)[4], bool stochastic, uint32_t f0,
                                             uint32_t unit, uint32_t epoch, uint32_t key_lo,
                                             uint32_t key_hi) {
  uint32_t h[4];
  if (stochastic) {
    uint32_t c[4] = {f0 >> 2, unit, epoch, 0u};
    philox4x32_10(c, key_lo, key_hi);
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = round_stochastic16<FMT>(x[e], c[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = round_nearest16<FMT>(x[e]);
  }
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

}  // namespace seed
