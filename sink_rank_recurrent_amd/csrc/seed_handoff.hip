// Handoff of shallow-form states between a state buffer and one contiguous
// transfer buffer.  At the end of the prefill a state is compressed to the
// sink plus rank-R factors (SEED figures and tables, Fig. 1 (a) caption,
// Table 1); a head in that form is 4 [d_k + (d_k + d_v) R] bytes in fp32
// (the byte account of Table 17 at w = 0), which is all a decode GPU needs.
//
// Packed layout: the selected requests one after another, each its heads in
// order, each head  a [d_k] fp32 | U columns 0..R-1 [R][d_k] | V columns
// 0..R-1 [R][d_v], the factors in the state's storage type.  Every segment
// is a multiple of 16 bytes, so one workgroup per (request, head) copies its
// head with 16-byte vectors in both directions.  An index outside [0, batch)
// selects nothing.
#include "seed_launch.h"

namespace seed {

namespace {

template <bool PACK>
__global__ __launch_bounds__(256) void handoff_kernel(float* __restrict__ a,
                                                      uint8_t* __restrict__ U,
                                                      uint8_t* __restrict__ V,
                                                      uint8_t* __restrict__ buf, const int* idx,
                                                      int batch, int heads, int d_k, int d_v,
                                                      int cap, int R, int fb) {
  const int i = blockIdx.x / heads;
  const int h = blockIdx.x - i * heads;
  const int b = idx[i];
  if (b < 0 || b >= batch) return;
  const size_t unit = (size_t)b * heads + h;
  // segment sizes in 16-byte vectors
  const int na = d_k / 4;
  const int nu = R * d_k * fb / 16;
  const int nv = R * d_v * fb / 16;
  const size_t ub = 16 * (size_t)(na + nu + nv);
  uint4* head = reinterpret_cast<uint4*>(buf + (size_t)blockIdx.x * ub);
  uint4* pa = reinterpret_cast<uint4*>(a + unit * d_k);
  uint4* pu = reinterpret_cast<uint4*>(U + unit * cap * d_k * fb);
  uint4* pv = reinterpret_cast<uint4*>(V + unit * cap * d_v * fb);
  for (int t = threadIdx.x; t < na + nu + nv; t += 256) {
    uint4* s = t < na ? pa + t : (t < na + nu ? pu + (t - na) : pv + (t - na - nu));
    if (PACK) head[t] = *s;
    else *s = head[t];
  }
}

// Join: handoff_kernel<false> into a batch of fp32 factor rings that holds
// r >= R columns, then columns R..r-1 of the slot's U and V set to zero (the
// batch appended them since its last compression; the joining request has
// no content there) and, for the lazily decayed form (gam_len > 0), the
// slot's decay product set to 1 (its columns are at true scale).
__global__ __launch_bounds__(256) void join_kernel(float* __restrict__ a, float* __restrict__ U,
                                                   float* __restrict__ V, float* __restrict__ gam,
                                                   const uint8_t* __restrict__ buf,
                                                   const int* slot, int batch, int heads, int d_k,
                                                   int d_v, int cap, int R, int r, int gam_len) {
  const int i = blockIdx.x / heads;
  const int h = blockIdx.x - i * heads;
  const int b = slot[i];
  if (b < 0 || b >= batch) return;
  const size_t unit = (size_t)b * heads + h;
  const int na = d_k / 4, nu = R * d_k / 4, nv = R * d_v / 4;
  const uint4* head = reinterpret_cast<const uint4*>(buf + (size_t)blockIdx.x * 16 * (na + nu + nv));
  uint4* pa = reinterpret_cast<uint4*>(a + unit * d_k);
  uint4* pu = reinterpret_cast<uint4*>(U + unit * cap * d_k);
  uint4* pv = reinterpret_cast<uint4*>(V + unit * cap * d_v);
  for (int t = threadIdx.x; t < na + nu + nv; t += 256) {
    uint4* d = t < na ? pa + t : (t < na + nu ? pu + (t - na) : pv + (t - na - nu));
    *d = head[t];
  }
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  const int zu = (r - R) * d_k / 4, zv = (r - R) * d_v / 4;
  for (int t = threadIdx.x; t < zu + zv; t += 256) {
    if (t < zu) pu[nu + t] = z;
    else pv[nv + t - zu] = z;
  }
  for (int t = threadIdx.x; t < gam_len; t += 256) gam[unit * gam_len + t] = 1.f;
}

}  // namespace

hipError_t launch_join(int batch, int heads, int d_k, int d_v, int cap, int R, int r, int gam_len,
                       int n_sel, const int* slot, const void* buf, float* a, float* U, float* V,
                       float* gam, hipStream_t stream) {
  if (n_sel == 0) return hipSuccess;
  const size_t blocks = (size_t)n_sel * heads;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(join_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, U, V, gam,
                     static_cast<const uint8_t*>(buf), slot, batch, heads, d_k, d_v, cap, R, r,
                     gam_len);
  return hipGetLastError();
}

hipError_t launch_handoff(bool pack, int batch, int heads, int d_k, int d_v, int cap, int R,
                          int factor_bytes, int n_sel, const int* idx, float* a, void* U, void* V,
                          void* buf, hipStream_t stream) {
  if (n_sel == 0) return hipSuccess;
  const size_t blocks = (size_t)n_sel * heads;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  if (pack) {
    hipLaunchKernelGGL(handoff_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       static_cast<uint8_t*>(U), static_cast<uint8_t*>(V),
                       static_cast<uint8_t*>(buf), idx, batch, heads, d_k, d_v, cap, R,
                       factor_bytes);
  } else {
    hipLaunchKernelGGL(handoff_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       static_cast<uint8_t*>(U), static_cast<uint8_t*>(V),
                       static_cast<uint8_t*>(buf), idx, batch, heads, d_k, d_v, cap, R,
                       factor_bytes);
  }
  return hipGetLastError();
}

}  // namespace seed
