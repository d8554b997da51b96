// Rounding of fp32 rank-R factors into the 16-bit storage of the kept
// columns: the store that ends a compression (SEED figures and tables,
// Table 4 and Table 9: fp16 or bf16 factors, rounded to nearest or
// stochastically at every compression), here for factors that come from
// elsewhere in fp32 -- the end-of-prefill compression or a handed-over
// state.  Each thread rounds four consecutive elements of one unit's block
// (U columns, then V columns) with the element numbering and generator
// words of the compression kernel, so the two produce the same patterns
// from the same fp32 values.
#include "seed_device.h"
#include "seed_launch.h"

namespace seed {

template <int FMT>
__global__ __launch_bounds__(256) void round_factors_kernel(
    const float* __restrict__ U, const float* __restrict__ V, uint16_t* __restrict__ Uk,
    uint16_t* __restrict__ Vk, int units, int R, int d_k, int d_v, int stochastic, uint32_t epoch,
    uint32_t key_lo, uint32_t key_hi) {
  const uint32_t nu = (uint32_t)R * d_k;                 // U elements per unit
  const uint32_t groups = (nu + (uint32_t)R * d_v) / 4;  // groups of four per unit
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)units * groups) return;
  const uint32_t unit = (uint32_t)(gid / groups);
  const uint32_t f0 = 4u * (uint32_t)(gid - (size_t)unit * groups);
  // d_k and d_v are multiples of 4: a group never straddles U and V
  const float* src;
  uint16_t* dst;
  if (f0 < nu) {
    src = U + (size_t)unit * nu + f0;
    dst = Uk + (size_t)unit * nu + f0;
  } else {
    const size_t nv = (size_t)R * d_v;
    src = V + unit * nv + (f0 - nu);
    dst = Vk + unit * nv + (f0 - nu);
  }
  const float4 t = *reinterpret_cast<const float4*>(src);
  const float x[4] = {t.x, t.y, t.z, t.w};
  *reinterpret_cast<uint2*>(dst) =
      round_pack4<FMT>(x, stochastic != 0, f0, unit, epoch, key_lo, key_hi);
}

hipError_t launch_round_factors(int store_fmt, int units, int R, int d_k, int d_v, const float* U,
                                const float* V, uint16_t* Uk, uint16_t* Vk, int stochastic,
                                uint32_t epoch, uint32_t key_lo, uint32_t key_hi,
                                hipStream_t stream) {
  const size_t threads = (size_t)units * ((size_t)R * (d_k + d_v) / 4);
  const size_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  if (store_fmt == kStoreBF16) {
    hipLaunchKernelGGL(round_factors_kernel<kStoreBF16>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, U, V, Uk, Vk, units, R, d_k, d_v, stochastic, epoch, key_lo, key_hi);
  } else if (store_fmt == kStoreF16) {
    hipLaunchKernelGGL(round_factors_kernel<kStoreF16>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, U, V, Uk, Vk, units, R, d_k, d_v, stochastic, epoch, key_lo, key_hi);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace seed
