// Statistics of dense states (seed_state_stats) on the compression kernel's
// tridiagonal eigensolver.
//
// What is computed (SEED figures and tables on thelatestinai.com: Fig. 3
// (e), (g), (h); Fig. 12 (f); Fig. 13 (a), (b), (d)).  Per unit: the sink
// split a = S vbar / |vbar|^2, C = S - a vbar^T; the energies |S|^2 (trace
// of S S^T), |a vbar^T|^2 = |a|^2 |vbar|^2 and |C|^2 (trace of C C^T); the
// whole spectra of S S^T and C C^T; the top eigenvector x_1 of S S^T and
// v* = S^T x_1, whose energy |v*|^2 (the Rayleigh quotient of x_1, second
// order in x_1's error) gives the top share; |cos(v*, vbar)|; the smallest
// ranks holding 90 % and 99 % of the content's energy and the share beyond
// rank R.  Record per unit (kStatFields floats): e_state, e_sink,
// e_content, sink share, top share, |cos(v*, vbar)|, rank90, rank99, share
// beyond R, then zeros.
//
// How: one workgroup of d_k threads per unit, thread t owning row and
// column t.  Each Gram (MFMA, from the rows of S, less the sink for C) is
// scaled by a power of two into unit range, reduced to tridiagonal T by
// Householder steps (the compression kernel's step, columns published
// through LDS), and every eigenvalue of T is found by its own thread by
// bisection on Sturm counts.  x_1 comes from inverse iteration on T and the
// reflectors.
#include "seed_compress_wave.h"

namespace seed {

namespace {

using wave::AddOp;
using wave::MaxOp;
using wave::MinOp;
using wave::block_reduce;
using wave::frcp;
using wave::fsqrt;
using wave::kEps;
using wave::load_row;
using wave::start_entry;

constexpr int kStatFields = 16;

// LDS layout (offsets in floats, every region a multiple of 4 floats)
template <int DK>
struct StatsLay {
  static constexpr int NMAX = DK;
  static constexpr int NW = DK / 64;
  static constexpr int NTH = 64 * NW;
  static constexpr int LDN = NMAX + 4;
  static constexpr int G = 0;                  // [NMAX][LDN] Gram, then reflectors (row k)
  static constexpr int CB = G + NMAX * LDN;    // [NTH] published column / solve factors
  static constexpr int VB = CB + NTH;          // [NTH]
  static constexpr int WB = VB + NTH;          // [NTH]
  static constexpr int TD = WB + NTH;          // [NMAX] diagonal of T
  static constexpr int TE = TD + NMAX;         // [NMAX] off-diagonal of T
  static constexpr int E2 = TE + NMAX;         // [NMAX] E2[i] = TE[i-1]^2
  static constexpr int TAU = E2 + NMAX;        // [NMAX]
  static constexpr int LAM = TAU + NMAX;       // [NMAX] eigenvalues, descending
  static constexpr int X1 = LAM + NMAX;        // [NMAX] top eigenvector
  static constexpr int AS = X1 + NMAX;         // [NMAX] sink coefficients
  static constexpr int VBS = AS + NMAX;        // [128] vbar
  static constexpr int PY = VBS + 128;         // [128] v*
  static constexpr int RED = PY + 128;         // [8][NW] cross-wave partials
  static constexpr int TOTAL = RED + 8 * NW + (8 * NW) % 4;
  static_assert(DK == 64 || DK == 128, "DK");
};

// Tridiagonalise the Gram in G (all NMAX columns) after scaling it by hs:
// T into TD, TE, E2 (scaled), the reflectors into the rows of G.
template <int NMAX, int NW>
__device__ __forceinline__ void tridiagonalise(float* G, float* CB, float* VB, float* WB,
                                               float* TD, float* TE, float* E2, float* TAU,
                                               float* RED, float hs) {
  constexpr int LDN = NMAX + 4;
  const int t = threadIdx.x;
  const int n = NMAX;
  float h[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) h[i] = G[i * LDN + t] * hs;
  __syncthreads();
  for (int k = 0; k + 2 < n; ++k) {
    if (t == k) {
#pragma unroll
      for (int i = 0; i < NMAX; i += 4)
        *reinterpret_cast<float4*>(CB + i) = make_float4(h[i], h[i + 1], h[i + 2], h[i + 3]);
    }
    __syncthreads();
    wave::tri_step<NMAX, NW, false>(h, k, CB[t], CB[k + 1], CB[k], t, true, VB, WB, G, TD, TE,
                                    TAU, RED);
  }
  if (t == n - 1) {
#pragma unroll
    for (int i = 0; i < NMAX; i += 4)
      *reinterpret_cast<float4*>(CB + i) = make_float4(h[i], h[i + 1], h[i + 2], h[i + 3]);
  }
  if (t == n - 2) {
#pragma unroll
    for (int i = 0; i < NMAX; i += 4)
      *reinterpret_cast<float4*>(VB + i) = make_float4(h[i], h[i + 1], h[i + 2], h[i + 3]);
  }
  __syncthreads();
  if (t == 0) {
    TD[n - 2] = VB[n - 2];
    TE[n - 2] = CB[n - 2];
    TD[n - 1] = CB[n - 1];
    TE[n - 1] = 0.f;
    TAU[n - 2] = 0.f;
    TAU[n - 1] = 0.f;
  }
  __syncthreads();
  E2[t] = t > 0 ? TE[t - 1] * TE[t - 1] : 0.f;
  __syncthreads();
}

// Eigenvalue number t (descending) of T by bisection on Sturm counts, one
// thread each, stopped at 4 eps |T|; returns it with |T| in tn.
template <int NMAX, int NW>
__device__ __forceinline__ float eigenvalue(const float* TD, const float* TE, const float* E2,
                                            float* RED, float& tn) {
  const int t = threadIdx.x;
  const float rad = fabsf(TE[t]) + (t > 0 ? fabsf(TE[t - 1]) : 0.f);
  float lo = block_reduce<NW>(TD[t] - rad, MinOp(), RED, 5);
  float hi = block_reduce<NW>(TD[t] + rad, MaxOp(), RED, 6);
  tn = fmaxf(fabsf(lo), fabsf(hi));
  const float pivmin = tn * 1e-30f + 1e-35f;
  lo -= 2.f * kEps * tn + pivmin;
  hi += 2.f * kEps * tn + pivmin;
  const int target = NMAX - 1 - t;             // ascending index
  const float tol = 4.f * kEps * tn + pivmin;
  for (int it = 0; it < 96 && hi - lo > tol; ++it) {
    const float x = 0.5f * (lo + hi);
    float q = 1.f;
    int cnt = 0;
    for (int i = 0; i < NMAX; ++i) {
      q = (TD[i] - x) - E2[i] * frcp(q);
      q = fabsf(q) < pivmin ? -pivmin : q;
      cnt += q < 0.f;
    }
    if (cnt > target) hi = x;
    else lo = x;
  }
  return 0.5f * (lo + hi);
}

// x_1 = the top eigenvector of the Gram: inverse iteration on T with the
// shift lam (thread 0; factors in CB, VB, WB), then back through the
// reflectors.  Leaves x_1 in X1.
template <int NMAX, int NW>
__device__ __forceinline__ void top_vector(float lam, float tn, const float* G, float* CB,
                                           float* VB, float* WB, const float* TD, const float* TE,
                                           const float* TAU, float* X1, float* RED) {
  constexpr int LDN = NMAX + 4;
  const int t = threadIdx.x;
  if (t == 0) {
    const float tiny = kEps * tn + 1e-30f;
    for (int i = 0; i < NMAX; ++i) X1[i] = start_entry(i, 0);
    for (int itn = 0; itn < 3; ++itn) {
      // factor T - lam I with partial pivoting while eliminating x
      float a = TD[0] - lam, b1 = TE[0], b2 = 0.f, rr = X1[0];
      for (int i = 0; i + 1 < NMAX; ++i) {
        const float lw = TE[i];
        const float ap = TD[i + 1] - lam;
        const float b1p = (i + 2 < NMAX) ? TE[i + 1] : 0.f;
        const float rp = X1[i + 1];
        const bool sw = fabsf(lw) > fabsf(a);
        const float pa = sw ? lw : ((a != 0.f) ? a : tiny);
        const float ipa = frcp(pa);
        CB[i] = ipa;
        VB[i] = sw ? ap : b1;
        WB[i] = sw ? b1p : b2;
        X1[i] = sw ? rp : rr;
        const float mm = (sw ? a : lw) * ipa;
        const float na = fmaf(-mm, sw ? ap : b1, sw ? b1 : ap);
        const float nb1 = fmaf(-mm, sw ? b1p : b2, sw ? b2 : b1p);
        const float nr = fmaf(-mm, sw ? rp : rr, sw ? rr : rp);
        a = na; b1 = nb1; b2 = 0.f; rr = nr;
      }
      CB[NMAX - 1] = frcp((a != 0.f) ? a : tiny);
      VB[NMAX - 1] = 0.f;
      WB[NMAX - 1] = 0.f;
      X1[NMAX - 1] = rr;
      float x1 = 0.f, x2 = 0.f, mx = 0.f;
      bool fin = true;
      for (int i = NMAX - 1; i >= 0; --i) {
        const float xi = (X1[i] - VB[i] * x1 - WB[i] * x2) * CB[i];
        X1[i] = xi;
        mx = fmaxf(mx, fabsf(xi));
        fin = fin && fabsf(xi) < 3.0e38f;
        x2 = x1;
        x1 = xi;
      }
      if (!fin || !(mx > 0.f)) {
        for (int i = 0; i < NMAX; ++i) X1[i] = start_entry(i, itn + 1);
        continue;
      }
      const float imx = frcp(mx);
      float nx = 0.f;
      for (int i = 0; i < NMAX; ++i) {
        X1[i] *= imx;
        nx = fmaf(X1[i], X1[i], nx);
      }
      const float inx = 1.f / sqrtf(nx);
      for (int i = 0; i < NMAX; ++i) X1[i] *= inx;
    }
  }
  __syncthreads();
  // x <- Q x, Q = H_0 H_1 ... H_{n-3} (reflector k in row k of G, entries > k)
  float xt = X1[t];
  __syncthreads();
  for (int k = NMAX - 3; k >= 0; --k) {
    const float vk = (t > k) ? G[k * LDN + t] : 0.f;   // reflector k: entries > k
    const float d = block_reduce<NW>(vk * xt, AddOp(), RED, (k & 1) ? 7 : 4);
    xt = fmaf(-TAU[k] * d, vk, xt);
  }
  X1[t] = xt;
  __syncthreads();
}

template <int DK, int DV>
__global__ __launch_bounds__(DK) void stats_wave_kernel(const float* __restrict__ S,
                                                        const float* __restrict__ vbar, int heads,
                                                        int R, float* __restrict__ rec,
                                                        float* __restrict__ specS,
                                                        float* __restrict__ specC) {
  using L = StatsLay<DK>;
  constexpr int NMAX = L::NMAX, NW = L::NW, LDN = L::LDN;
  extern __shared__ float4 smem4[];
  float* const sm = reinterpret_cast<float*>(smem4);
  float* const G = sm + L::G;
  float* const CB = sm + L::CB;
  float* const VB = sm + L::VB;
  float* const WB = sm + L::WB;
  float* const TD = sm + L::TD;
  float* const TE = sm + L::TE;
  float* const E2 = sm + L::E2;
  float* const TAU = sm + L::TAU;
  float* const LAM = sm + L::LAM;
  float* const X1 = sm + L::X1;
  float* const AS = sm + L::AS;
  float* const VBS = sm + L::VBS;
  float* const PY = sm + L::PY;
  float* const RED = sm + L::RED;
  const int t = threadIdx.x;
  const size_t ub = blockIdx.x;
  const float* const Sh = S + ub * DK * DV;
  float* const out = rec + ub * kStatFields;

  for (int e = t; e < DV; e += NMAX) VBS[e] = vbar[(size_t)(ub % heads) * DV + e];
  __syncthreads();
  float nv2 = 0.f;
  for (int e = 0; e < DV; ++e) nv2 = fmaf(VBS[e], VBS[e], nv2);
  {
    float p0 = 0.f, p1 = 0.f;
    for (int e = 0; e < DV; e += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(Sh + (size_t)t * DV + e);
      p0 = fmaf(x4.x, VBS[e], p0);
      p1 = fmaf(x4.y, VBS[e + 1], p1);
      p0 = fmaf(x4.z, VBS[e + 2], p0);
      p1 = fmaf(x4.w, VBS[e + 3], p1);
    }
    AS[t] = nv2 > 0.f ? (p0 + p1) / nv2 : 0.f;
  }
  __syncthreads();
  float na = 0.f;
  for (int i = 0; i < NMAX; ++i) na = fmaf(AS[i], AS[i], na);
  const float e_sink = na * nv2;

  auto scol = [&](int j) -> const float* { return Sh + (size_t)j * DV; };
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0)
      wave::gram<NMAX, NW, DV, false, kStoreF32, 0>(scol, nullptr, NMAX, G, nullptr, nullptr,
                                                    false);
    else
      wave::gram<NMAX, NW, DV, false, kStoreF32, 0, decltype(scol), true>(
          scol, nullptr, NMAX, G, nullptr, nullptr, false, AS, VBS);
    __syncthreads();
    // the trace, summed by every thread in the same order
    float tr = 0.f;
    for (int i = 0; i < NMAX; ++i) tr += G[i * LDN + i];
    // scale H into unit range by a power of two (exact)
    const float mxd = block_reduce<NW>(G[t * LDN + t], MaxOp(), RED, 2);
    float hs = 1.f;
    if (mxd > 0.f && mxd < 3.0e38f) {
      int ex;
      frexpf(mxd, &ex);
      hs = ldexpf(1.f, -ex);
    }
    tridiagonalise<NMAX, NW>(G, CB, VB, WB, TD, TE, E2, TAU, RED, hs);
    float tn;
    const float lam = eigenvalue<NMAX, NW>(TD, TE, E2, RED, tn);
    const float ihs = 1.f / hs;
    LAM[t] = lam * ihs;
    float* spec = pass == 0 ? specS : specC;
    if (spec != nullptr) spec[ub * DK + t] = lam * ihs;
    __syncthreads();
    if (pass == 0) {
      top_vector<NMAX, NW>(LAM[0] * hs, tn, G, CB, VB, WB, TD, TE, TAU, X1, RED);
      // v* = S^T x_1 in value space
      for (int e = t; e < DV; e += NMAX) {
        float y = 0.f;
        for (int j = 0; j < NMAX; ++j) y = fmaf(Sh[(size_t)j * DV + e], X1[j], y);
        PY[e] = y;
      }
      __syncthreads();
      if (t == 0) {
        float nn = 0.f, dot = 0.f;
        for (int e = 0; e < DV; ++e) {
          nn = fmaf(PY[e], PY[e], nn);
          dot = fmaf(PY[e], VBS[e], dot);
        }
        out[0] = tr;
        out[1] = e_sink;
        out[3] = tr > 0.f ? e_sink / tr : 0.f;
        out[4] = tr > 0.f ? nn / tr : 0.f;
        out[5] = (nn > 0.f && nv2 > 0.f) ? fabsf(dot) / sqrtf(nn * nv2) : 0.f;
        for (int f = 9; f < kStatFields; ++f) out[f] = 0.f;
      }
    } else if (t == 0) {
      float tot = 0.f;
      for (int i = 0; i < NMAX; ++i) tot += fmaxf(LAM[i], 0.f);
      int r90 = 0, r99 = 0;
      float c = 0.f, beyond = 0.f;
      for (int i = 0; i < NMAX; ++i) {
        const float li = fmaxf(LAM[i], 0.f);
        c += li;
        if (r90 == 0 && tot > 0.f && c >= 0.90f * tot) r90 = i + 1;
        if (r99 == 0 && tot > 0.f && c >= 0.99f * tot) r99 = i + 1;
        if (i >= R) beyond += li;
      }
      out[2] = tr;
      out[6] = (float)r90;
      out[7] = (float)r99;
      out[8] = tot > 0.f ? beyond / tot : 0.f;
    }
    __syncthreads();
  }
}

template <int DK, int DV>
hipError_t stats_go(int units, int heads, int R, const float* S, const float* vbar, float* rec,
                    float* specS, float* specC, hipStream_t s) {
  const size_t bytes = 4 * (size_t)StatsLay<DK>::TOTAL;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(stats_wave_kernel<DK, DV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((stats_wave_kernel<DK, DV>), dim3(units), dim3(DK), bytes, s, S, vbar, heads,
                     R, rec, specS, specC);
  return hipGetLastError();
}

}  // namespace

int stat_fields() { return kStatFields; }

size_t stats_lds_bytes(int d_k, int /*R*/) {
  return d_k == 128 ? 4 * (size_t)StatsLay<128>::TOTAL : 4 * (size_t)StatsLay<64>::TOTAL;
}

hipError_t launch_state_stats(int batch, int heads, int d_k, int d_v, int R, const float* S,
                              const float* vbar, float* rec, float* specS, float* specC,
                              hipStream_t stream) {
  const int units = batch * heads;
  if (d_k == 128 && d_v == 128)
    return stats_go<128, 128>(units, heads, R, S, vbar, rec, specS, specC, stream);
  if (d_k == 128 && d_v == 64)
    return stats_go<128, 64>(units, heads, R, S, vbar, rec, specS, specC, stream);
  if (d_k == 64 && d_v == 64)
    return stats_go<64, 64>(units, heads, R, S, vbar, rec, specS, specC, stream);
  return hipErrorInvalidValue;
}

}  // namespace seed
