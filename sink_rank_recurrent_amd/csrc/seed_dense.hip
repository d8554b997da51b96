// Dense-state baseline: one step of the head's own recurrence on the full
// d_k x d_v state, then the read-out of the updated state.
//   Gated DeltaNet:       S' = g S + beta k (v - g S^T k)^T
//   Kimi Delta Attention: T = Diag(g) S;  S' = T + beta k (v - T^T k)^T
//   Mamba-2:              S' = g S + k v^T
//   o = S'^T q
// (These are the literal forms g (I - beta k k^T) S + beta k v^T and
// (I - beta k k^T) Diag(g) S + beta k v^T multiplied out; SEED summary on
// picx.dev names the three updates under "Exact Update (Lemma 2)".)
//
// Mapping: one 256-thread workgroup per (request, head).  A row of S (one
// key channel, d_v floats) is spread over d_v/4 lanes with one 16-byte
// access each; the workgroup covers 256/(d_v/4) rows at a time and each
// thread keeps d_k/(256/(d_v/4)) rows in registers, so S is read once and
// written once, both non-temporally (a state is not reused before the other
// layers' states have streamed through).  The two column sums (S^T k, then
// S'^T q) are combined across row groups through LDS.
#include "seed_device.h"
#include "seed_launch.h"

namespace seed {

template <int RULE, int DK, int DV, typename IN_T>
__global__ __launch_bounds__(256) void dense_step_kernel(
    float* __restrict__ S, const IN_T* __restrict__ q, const IN_T* __restrict__ k,
    const IN_T* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ o) {
  constexpr int LV = DV / 4;     // lanes per row
  constexpr int RG = 256 / LV;   // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(RPT * RG == DK, "rows must tile");
  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int rg = tid / LV;
  const int lc = tid % LV;
  const size_t ub = (size_t)unit;
  float* Sh = S + ub * DK * DV;

  float s[RPT][4];
#pragma unroll
  for (int m = 0; m < RPT; ++m) load_vec_nt<4>(Sh + (size_t)(rg + RG * m) * DV + lc * 4, s[m]);
  float kr[RPT], qr[RPT], gr[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    kr[m] = load_scalar(k + ub * DK + row);
    qr[m] = load_scalar(q + ub * DK + row);
    if constexpr (RULE == kKDA) gr[m] = g[ub * DK + row];
  }
  float gs = 1.f, bt = 1.f;
  if constexpr (RULE != kKDA) gs = g[ub];
  if constexpr (RULE != kMAMBA2) bt = beta[ub];
  float vv[4];
  load_vec<4>(v + ub * DV + lc * 4, vv);

  __shared__ float red[RG][DV];
  if constexpr (RULE != kMAMBA2) {
    // w = S^T k (Gated DeltaNet) or (Diag(g) S)^T k (Kimi Delta Attention)
    float pw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const float coef = (RULE == kKDA) ? kr[m] * gr[m] : kr[m];
#pragma unroll
      for (int c = 0; c < 4; ++c) pw[c] += coef * s[m][c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) red[rg][lc * 4 + c] = pw[c];
    __syncthreads();
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) wv[c] += red[j][lc * 4 + c];
    }
    __syncthreads();  // red is reused below
    // residual written along k
    float dv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dv[c] = (RULE == kKDA) ? vv[c] - wv[c] : vv[c] - gs * wv[c];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const float decay = (RULE == kKDA) ? gr[m] : gs;
      const float bk = bt * kr[m];
#pragma unroll
      for (int c = 0; c < 4; ++c) s[m][c] = decay * s[m][c] + bk * dv[c];
    }
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
#pragma unroll
      for (int c = 0; c < 4; ++c) s[m][c] = gs * s[m][c] + kr[m] * vv[c];
    }
  }

#pragma unroll
  for (int m = 0; m < RPT; ++m) store_vec_nt<4>(Sh + (size_t)(rg + RG * m) * DV + lc * 4, s[m]);

  // o = S'^T q
  float po[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
#pragma unroll
    for (int c = 0; c < 4; ++c) po[c] += qr[m] * s[m][c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[rg][lc * 4 + c] = po[c];
  __syncthreads();
  if (rg == 0) {
    float ov[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] += red[j][lc * 4 + c];
    }
    store_vec<4>(o + ub * DV + lc * 4, ov);
  }
}

namespace {

template <int RULE, int DK, int DV, typename IN_T>
hipError_t dense_go(int units, float* S, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* o, hipStream_t s) {
  hipLaunchKernelGGL((dense_step_kernel<RULE, DK, DV, IN_T>), dim3(units), dim3(256), 0, s, S,
                     static_cast<const IN_T*>(q), static_cast<const IN_T*>(k),
                     static_cast<const IN_T*>(v), g, beta, o);
  return hipGetLastError();
}

template <int RULE, typename IN_T>
hipError_t dense_dims(int units, int d_k, int d_v, float* S, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, float* o, hipStream_t s) {
  if (d_k == 128 && d_v == 128) return dense_go<RULE, 128, 128, IN_T>(units, S, q, k, v, g, beta, o, s);
  if (d_k == 128 && d_v == 64) return dense_go<RULE, 128, 64, IN_T>(units, S, q, k, v, g, beta, o, s);
  if (d_k == 64 && d_v == 64) return dense_go<RULE, 64, 64, IN_T>(units, S, q, k, v, g, beta, o, s);
  return hipErrorInvalidValue;
}

template <int RULE>
hipError_t dense_dtype(bool bf16, int units, int d_k, int d_v, float* S, const void* q,
                       const void* k, const void* v, const float* g, const float* beta, float* o,
                       hipStream_t s) {
  if (bf16) return dense_dims<RULE, bf16_t>(units, d_k, d_v, S, q, k, v, g, beta, o, s);
  return dense_dims<RULE, float>(units, d_k, d_v, S, q, k, v, g, beta, o, s);
}

}  // namespace

hipError_t launch_dense(int rule, bool in_bf16, int batch, int heads, int d_k, int d_v, float* S,
                        const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float* o, hipStream_t stream) {
  const int units = batch * heads;
  switch (rule) {
    case kGDN: return dense_dtype<kGDN>(in_bf16, units, d_k, d_v, S, q, k, v, g, beta, o, stream);
    case kKDA: return dense_dtype<kKDA>(in_bf16, units, d_k, d_v, S, q, k, v, g, beta, o, stream);
    case kMAMBA2:
      return dense_dtype<kMAMBA2>(in_bf16, units, d_k, d_v, S, q, k, v, g, beta, o, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace seed
