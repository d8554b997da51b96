// Compression of the factors to rank R with one or two wave64 per
// (request, head): the kernel template, instantiated per head shape by
// seed_compress_wave_<d_k>x<d_v>.hip.
//
// Mathematics (SEED figures and tables on thelatestinai.com, Fig. 1 (b)
// caption: the content U V^T is replaced by its best rank-R approximation,
// the sink untouched).  With U^T U = R_U^T R_U (n = R + W columns),
//     H = R_U (V^T V) R_U^T = X diag(s^2) X^T,
//     U' = U R_U^-1 X_R,   V' = V R_U^T X_R,
// and U' V'^T is the truncation of U V^T to its R largest singular values.
// Phases:
//   A  Gram matrices U^T U and V^T V by v_mfma_f32_16x16x4f32;
//   B  Cholesky with diagonal pivoting of the column-equilibrated U^T U
//      (P^T D^-1 U^T U D^-1 P = R~^T R~ over the kept columns, R_U = R~ D),
//      thread t owning column t;
//   C  H = R~ (D V^T V D) R~^T by two in-place MFMA products;
//   D  Householder reduction of H to a tridiagonal T, thread t owning
//      column t of H in registers; the reflectors go to LDS rows;
//   E  the R largest eigenvalues of T by multisection on Sturm counts;
//   F  their eigenvectors by inverse iteration (pivoted tridiagonal solve),
//      re-orthogonalised inside runs of close eigenvalues, then one modified
//      Gram-Schmidt pass;
//   G  back-transform through the reflectors (X_R = Q Y);
//   H  P2 = D R~^T X_R (MFMA) and T' = D^-1 P R~^-1 X_R (back substitution
//      in pivot order);
//   I  U' = U T' and V' = V P2 by MFMA, written in place.
// Every LDS offset is a compile-time constant, so accesses use immediate
// offsets and 16-byte vector forms.  With one wave the workgroup barriers
// only order LDS traffic inside the wave.
#pragma once

#include <atomic>

#include "seed_device.h"
#include "seed_launch.h"

namespace seed {
namespace wave {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kEps = 1.1920928955078125e-7f;   // 2^-23
// Dependent-column threshold of the pivoted Cholesky (relative to the unit
// diagonal of the equilibrated Gram): the columns left when the largest
// remaining diagonal is at most this have parts orthogonal to the kept ones
// below sqrt(kPivTol) = 3.2e-4 of their norms, and are dropped.
constexpr float kPivTol = 1e-7f;
constexpr float kMinNormal = 1.17549435e-38f;      // smallest normal fp32
// Eigenvalues closer than kClusterTol |T| form a run whose vectors are
// computed one after another, each re-orthogonalised against the earlier
// ones of its run.
constexpr float kClusterTol = 1e-5f;
constexpr int kInvIters = 2;
// Eigenvalues below kEigFloor eps |T| are resolved only to that absolute
// accuracy (they sit at the rounding level of T's entries).
constexpr float kEigFloor = 1e-3f;
// T is padded to NMAX rows with this diagonal and zero couplings; the padded
// entries of every solve are exactly 0.
constexpr float kPadDiag = 1.0e30f;

// ---------------------------------------------------------------------------
// reductions

// Sum / min / max over the 64 lanes of a wave, returned to every lane: DPP
// butterflies inside each row of 16 lanes, then one readlane per row.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}
struct AddOp { __device__ float operator()(float a, float b) const { return a + b; } };
struct MinOp { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// The same over the NW waves of the workgroup; `red` holds one slot of NW
// partials per call site, and every slot is separated from its next use by
// a barrier of the surrounding loop.
template <int NW, typename Op>
__device__ __forceinline__ float block_reduce(float x, Op op, float* red, int slot) {
  const float s = wave_reduce(x, op);
  if constexpr (NW == 1) {
    return s;
  } else {
    if ((threadIdx.x & 63) == 0) red[slot * NW + (threadIdx.x >> 6)] = s;
    __syncthreads();
    float r = red[slot * NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = op(r, red[slot * NW + w]);
    return r;
  }
}

template <int NW>
__device__ __forceinline__ bool block_all(bool p, float* red, int slot) {
  if constexpr (NW == 1) {
    return __all(p);
  } else {
    return block_reduce<NW>(p ? 1.f : 0.f, MinOp(), red, slot) > 0.5f;
  }
}

// The lowest thread of the workgroup whose predicate holds, returned to
// every thread (NTH if there is none).  With two waves the per-wave
// candidates meet in slot 7 of `red`, separated from its next use by a
// barrier of the surrounding loop.
template <int NW>
__device__ __forceinline__ int block_first(bool p, float* red) {
  const unsigned long long b = __ballot(p);
  const int w = threadIdx.x >> 6;
  const int mine = b ? 64 * w + __builtin_ctzll(b) : 64 * NW;
  if constexpr (NW == 1) {
    return mine;
  } else {
    if ((threadIdx.x & 63) == 0) red[7 * NW + w] = __int_as_float(mine);
    __syncthreads();
    int best = __float_as_int(red[7 * NW]);
#pragma unroll
    for (int i = 1; i < NW; ++i) best = min(best, __float_as_int(red[7 * NW + i]));
    return best;
  }
}

// Sum over groups of P consecutive lanes (P = 2 or 4), returned to the group.
template <int P>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
  if constexpr (P == 4)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
  return x;
}

// Lane `own` of each group of P consecutive lanes, broadcast to the group.
template <int P, int own>
__device__ __forceinline__ float group_bcast(float x) {
  constexpr int ctrl = (P == 4) ? (own | (own << 2) | (own << 4) | (own << 6))
                                : (own | (own << 2) | ((2 + own) << 4) | ((2 + own) << 6));
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false));
}

// x[0..N) = p[0..N), p 16-byte aligned, read with 16-byte loads.
template <int N>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
  }
}

__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float frsq(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float fsqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

// Deterministic start vector of inverse iteration, entries in [0.5, 1.5).
__device__ __forceinline__ float start_entry(int i, int c) {
  uint32_t h = (uint32_t)(i + 1) * 2654435761u ^ (uint32_t)(c + 1) * 2246822519u;
  h ^= h >> 13;
  h *= 3266489917u;
  h ^= h >> 16;
  return (float)(h & 0xFFFFu) * (1.0f / 65536.0f) + 0.5f;
}

// ---------------------------------------------------------------------------
// LDS layout (offsets in floats; every region a multiple of 4 floats)

// NO_RB: the conversion's layout, which has no R~ (and no decay product).
template <int NMAX, int RMAX, bool NO_RB = false>
struct Lay {
  static constexpr int NW = (NMAX + 63) / 64;     // waves per unit
  static constexpr int NTH = 64 * NW;
  static constexpr int LDN = NMAX + 4;             // row stride: 16-byte aligned rows
  static constexpr int PARTS = NTH / RMAX < 4 ? NTH / RMAX : 4;   // lanes per eigenvector
  static constexpr int NACT = RMAX * PARTS;        // threads holding eigenvector rows
  static constexpr int CH = NMAX / PARTS;          // rows per lane
  // one wave keeps two of the three solve factors of phase F in registers
  static constexpr bool FREG = NW == 1;
  // The regions used from phase D on ("late") go into G, which is free once
  // H is in registers, when they fit (the compression); else after RB.
  static constexpr int LATE = 2 * NMAX * RMAX + (FREG ? 0 : 2 * NMAX * RMAX) + 6 * NMAX + 3 * RMAX;
  // the published vectors and the two scales of phase H (see T0 below)
  static constexpr int TAILN = 3 * NTH + 2 * NMAX;
  // Two-wave compressions keep G unpadded (row stride NMAX) when the late
  // regions and that tail still fit: at n = 80 that brings a unit to 53.2
  // KB, so three units share a CU.  The padding only spreads the banks of
  // G's transposed stores and tile reads (phases A and C, once per
  // compression).
  static constexpr bool GPACK = !NO_RB && NW == 2 && LATE + TAILN <= NMAX * NMAX;
  static constexpr int LDG = GPACK ? NMAX : LDN;   // row stride of G
  static constexpr int G = 0;                      // [NMAX][LDG] Grams, Z, H (the conversion: then reflectors)
  // [NMAX][LDN] R~ in pivot order, RB[p LDN + i] = R~[i][PIV[p]] (i <= p),
  // and reflector k in row k at entries > k
  static constexpr int RB = G + NMAX * LDG;
  static constexpr bool COMPACT = !NO_RB && LATE <= NMAX * LDG;
  static constexpr int L0 = COMPACT ? G : RB + (NO_RB ? 0 : NMAX * LDN);
  static constexpr int XR = L0;                    // [NMAX][RMAX] eigenvectors, Y, then T'
  static constexpr int FA = XR + NMAX * RMAX;      // [NMAX][RMAX] reciprocal pivots of phase F, then P2
  static constexpr int FB = FA + NMAX * RMAX;      // [NMAX][RMAX] x 2 (not with FREG): the superdiagonals
  static constexpr int FC = FB + (FREG ? 0 : NMAX * RMAX);
  static constexpr int TD = FC + (FREG ? 0 : NMAX * RMAX);   // [NMAX] diagonal of T
  static constexpr int TE = TD + NMAX;             // [NMAX] off-diagonal of T
  static constexpr int E2 = TE + NMAX;             // [NMAX] E2[i] = TE[i-1]^2
  static constexpr int TAU = E2 + NMAX;            // [NMAX]
  static constexpr int CB2 = TAU + NMAX;           // [2][NMAX] Gram-Schmidt pivot (double buffer)
  static constexpr int LAM = CB2 + 2 * NMAX;       // [RMAX] eigenvalues (descending)
  static constexpr int RNK = LAM + RMAX;           // [RMAX] round of each vector (int)
  static constexpr int STA = RNK + RMAX;           // [RMAX] first index of its run (int)
  static constexpr int LEND = STA + RMAX;
  static constexpr int BPT = XR;                   // [4 NTH] bisection points (XR, FA free then)
  static constexpr int BFL = XR + 4 * NTH;         // [4 NTH] their flags (int)
  // the regions used before phase D or throughout ("early")
  static constexpr int E0 = COMPACT ? RB + NMAX * LDN : LEND;
  // The published vectors and the two scales of phase H go into the tail of
  // G past the late regions when they fit there: G holds nothing during
  // phase B (each thread has its Gram column in registers) and nothing
  // there from phase D on, and the scales are kept in registers until D
  // stores them.  That keeps a unit at n = 48, R = 16 within 20 KB, so
  // eight units share a CU.
  static constexpr bool TAIL = COMPACT && LEND + TAILN <= G + NMAX * LDG;
  static constexpr int T0 = TAIL ? LEND : E0;
  static constexpr int CB = T0;                    // [NTH] published column
  static constexpr int VB = CB + NTH;              // [NTH] Householder vector
  static constexpr int WB = VB + NTH;              // [NTH] rank-2 update vector
  static constexpr int IDV = WB + NTH;             // [NMAX] 1/d (stored in phase D)
  static constexpr int IRD = IDV + NMAX;           // [NMAX] 1/R~[i][i] (stored in phase D)
  static constexpr int DV = TAIL ? E0 : IRD + NMAX;   // [NMAX] column norms d of U
  static constexpr int PIV = DV + NMAX;            // [NMAX] column at each pivot position (int)
  // decay product per key row (lazy form), 128 entries: in the 4 padding
  // columns of the rows of RB (never read or written otherwise) when they
  // hold 128 entries, else in a region of its own
  static constexpr bool GS_PAD = !NO_RB && 4 * NMAX >= 128;
  static constexpr int GS = PIV + NMAX;
  static constexpr int RED = GS + (GS_PAD ? 0 : 128);   // [8][NW] cross-wave partials
  static constexpr int MISC = RED + 8 * NW + (8 * NW) % 4;
  static constexpr int TOTAL = MISC + 4;
  static_assert(NMAX % 16 == 0 && NMAX <= 128, "NMAX");
  static_assert(8 * NTH <= 2 * NMAX * RMAX, "bisection points fit in XR and FA");
  static_assert(RMAX == 16 || RMAX == 32, "RMAX");
  static_assert(!COMPACT || LEND <= G + NMAX * LDG, "late regions fit in G");
};

// Waves per SIMD the compiler plans registers for: two where a
// compression's LDS lets more than four one-wave units, or three two-wave
// units (in 512-byte allocation granules), share a CU; one otherwise (the
// conversion, at n = d_k, keeps the whole register file).
template <int NMAX, int RMAX, bool NO_RB>
constexpr int wave_min_waves() {
  using L = Lay<NMAX, RMAX, NO_RB>;
  constexpr size_t granules = (4 * (size_t)L::TOTAL + 511) / 512;
  return (!NO_RB && ((L::NW == 1 && 4 * L::TOTAL <= 32 * 1024) ||
                     (L::NW == 2 && 3 * 512 * granules <= 160 * 1024))) ? 2 : 1;
}

// ---------------------------------------------------------------------------
// A: G[i][j] = s_ij sum_e X[e][i] X[e][j] for i, j < NMAX (zero beyond n),
// s_ij = d_i d_j when SCALE, else 1.  Column j < KR of X is the 16-bit
// column j of Xk (format FMT), any other column is fp32 at colf(j); each
// holds D entries.  MFMA 16x16x4: lane l feeds column 16 t + l % 16 of
// tile t at the k-slot l / 16.  Wave w sums e over [w D / NW, (w + 1) D / NW),
// slot kk over its quarter of that range; with two waves the partial sums
// meet in LDS (wave 1 stores, wave 0 adds and stores the total).  If rs is
// not NULL, row e of X is first multiplied by rs[e] (rs_per_row) or by rs[0].
// With CORR, column j is first replaced by X_j - ca[j] cb (the content of a
// dense state: a row of S less its sink).  With PERM, entry (i, j) is that of
// columns perm[i] and perm[j] (perm a permutation of 0 .. NMAX-1 that keeps
// 0 .. n-1 among themselves), scaled by dv[perm[i]] dv[perm[j]].
template <int NMAX, int NW, int D, bool SCALE, int FMT, int KR, typename ColF,
          bool CORR = false, bool PERM = false, int LDG = NMAX + 4>
__device__ __forceinline__ void gram(ColF colf, const uint16_t* __restrict__ Xk,
                                     int n, float* __restrict__ G,
                                     const float* __restrict__ dv, const float* __restrict__ rs,
                                     bool rs_per_row, const float* __restrict__ ca = nullptr,
                                     const float* __restrict__ cb = nullptr,
                                     const int* __restrict__ perm = nullptr) {
  constexpr int NT = NMAX / 16;
  constexpr int NP = NT * (NT + 1) / 2;
  constexpr int KPL = D / (4 * NW);
  // k-slots per load round: all of a lane's slots at once when they fit in
  // 96 registers (one HBM round trip instead of two), else chunks
  constexpr int KC0 = ((NT > 4) ? 8 : 16) < KPL ? ((NT > 4) ? 8 : 16) : KPL;
  constexpr int KC = (NT * KPL <= 96) ? KPL : KC0;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ci = l & 15, kk = l >> 4;
  f4v acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < KPL; s0 += KC) {
    float x[NT][KC];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int pos = t * 16 + ci;
      const int col = PERM ? perm[pos] : pos;
      const int off = (w * 4 + kk) * KPL + s0;
      if ((FMT == kStoreBF16 || FMT == kStoreF16) && col < n && col < KR) {
        const uint16_t* src = Xk + (size_t)col * D + off;
#pragma unroll
        for (int q = 0; q < KC / 4; ++q) {
          float y[4];
          load_vec16<FMT, 4>(src + 4 * q, y);
          x[t][4 * q + 0] = y[0]; x[t][4 * q + 1] = y[1];
          x[t][4 * q + 2] = y[2]; x[t][4 * q + 3] = y[3];
        }
      } else if (col < n) {
        const float* src = colf(col) + off;
#pragma unroll
        for (int q = 0; q < KC / 4; ++q) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + 4 * q);
          x[t][4 * q + 0] = v4.x; x[t][4 * q + 1] = v4.y;
          x[t][4 * q + 2] = v4.z; x[t][4 * q + 3] = v4.w;
        }
      } else {
#pragma unroll
        for (int s = 0; s < KC; ++s) x[t][s] = 0.f;
      }
      if constexpr (CORR) {
        // column col less ca[col] cb (entries off .. off + KC of cb)
        if (col < n) {
          const float c0 = ca[col];
#pragma unroll
          for (int q = 0; q < KC / 4; ++q) {
            const float4 b4 = *reinterpret_cast<const float4*>(cb + off + 4 * q);
            x[t][4 * q + 0] = fmaf(-c0, b4.x, x[t][4 * q + 0]);
            x[t][4 * q + 1] = fmaf(-c0, b4.y, x[t][4 * q + 1]);
            x[t][4 * q + 2] = fmaf(-c0, b4.z, x[t][4 * q + 2]);
            x[t][4 * q + 3] = fmaf(-c0, b4.w, x[t][4 * q + 3]);
          }
        }
      }
    }
    if (rs != nullptr) {
      float sc[KC];
      if (rs_per_row) {
        const float* src = rs + (w * 4 + kk) * KPL + s0;
#pragma unroll
        for (int q = 0; q < KC / 4; ++q) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + 4 * q);
          sc[4 * q + 0] = v4.x; sc[4 * q + 1] = v4.y; sc[4 * q + 2] = v4.z; sc[4 * q + 3] = v4.w;
        }
      } else {
        const float r0 = rs[0];
#pragma unroll
        for (int s = 0; s < KC; ++s) sc[s] = r0;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < KC; ++s) x[t][s] *= sc[s];
    }
    int p = 0;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = I; J < NT; ++J) {
#pragma unroll
        for (int s = 0; s < KC; ++s)
          acc[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[I][s], x[J][s], acc[p], 0, 0, 0);
        ++p;
      }
  }
  // lane l holds D[4 (l/16) + r][l % 16] of each 16 x 16 tile
  if constexpr (NW > 1) {
    if (w == 1) {
      int p = 0;
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I; J < NT; ++J) {
#pragma unroll
          for (int r = 0; r < 4; ++r) G[(I * 16 + 4 * kk + r) * LDG + J * 16 + ci] = acc[p][r];
          ++p;
        }
    }
    __syncthreads();
    if (w == 0) {
      // every partial is read before any total is stored (the diagonal
      // tiles store transposed positions that other lanes still read)
      int p = 0;
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I; J < NT; ++J) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[p][r] += G[(I * 16 + 4 * kk + r) * LDG + J * 16 + ci];
          ++p;
        }
    }
  }
  if (w == 0) {
    int p = 0;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = I; J < NT; ++J) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = I * 16 + 4 * kk + r, j = J * 16 + ci;
          float v = acc[p][r];
          if constexpr (SCALE) v *= dv[PERM ? perm[i] : i] * dv[PERM ? perm[j] : j];
          G[i * LDG + j] = v;
          G[j * LDG + i] = v;
        }
        ++p;
      }
  }
}

// Rows i updated by a step at index j: whole aligned groups of 4 rows when
// j is a compile-time constant (fully unrolled loops), so that the 16-byte
// LDS reads stay whole; whole 8-row blocks (one uniform branch each)
// otherwise.  Rows <= j of a group are updated harmlessly.
template <bool STATIC>
__device__ __forceinline__ bool live_row(int i, int j) {
  if constexpr (STATIC) return (i | 3) > j;
  else return (i | 7) > j;
}

// D, one Householder step k: thread t owns column t of H in h, hk is
// H[t][k], alpha = H[k+1][k], dkk = H[k][k].  Records T's row k and the
// reflector (row k of RS, entries > k), then H <- H - v w^T - w v^T on the
// rows > k (rows <= k of a column are never read again).
template <int NMAX, int NW, bool STATIC>
__device__ __forceinline__ void tri_step(float (&h)[NMAX], int k, float hk, float alpha, float dkk,
                                         int t, bool act, float* VB, float* WB, float* RS,
                                         float* TD, float* TE, float* TAU, float* RED) {
  constexpr int LDN = NMAX + 4;
  const float xn2 = block_reduce<NW>(t > k + 1 ? hk * hk : 0.f, AddOp(), RED, 0);
  float tau = 0.f, beta = alpha, sc = 0.f;
  // a column whose sub-subdiagonal part squares to a subnormal (below
  // 1e-19 of H's scale, itself near 1) is taken as already reduced
  if (xn2 >= kMinNormal) {
    const float nrm = fsqrt(fmaf(alpha, alpha, xn2));
    beta = alpha >= 0.f ? -nrm : nrm;
    tau = (beta - alpha) * frcp(beta);
    sc = frcp(alpha - beta);
  }
  const float vl = (t > k + 1) ? hk * sc : (t == k + 1 ? 1.f : 0.f);
  if (t == 0) {
    TD[k] = dkk;
    TE[k] = beta;
    TAU[k] = tau;
  }
  if (act) VB[t] = vl;
  // reflector k in row k of RS at entries t > k (its zeros at t <= k are
  // not stored: readers take them as zero)
  if (act && t > k) RS[k * LDN + t] = vl;
  __syncthreads();
  // v is read whole before the first use (it stays live for the update)
  float vv[NMAX];
  load_row<NMAX>(VB, vv);
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int b = 0; b < NMAX / 8; ++b) {
    if (live_row<STATIC>(8 * b + 7, k)) {
#pragma unroll
      for (int i = 8 * b; i < 8 * b + 8; ++i) {
        if (live_row<STATIC>(i, k)) {
          if (i & 1) pb = fmaf(h[i], vv[i], pb);
          else pa = fmaf(h[i], vv[i], pa);
        }
      }
    }
  }
  const float pl = (pa + pb) * tau;
  const float K = -0.5f * tau * block_reduce<NW>(pl * vl, AddOp(), RED, 1);
  const float wl = fmaf(K, vl, pl);
  if (act) WB[t] = wl;
  __syncthreads();
  if constexpr (NMAX <= 64) {
    float wr[NMAX];
    load_row<NMAX>(WB, wr);
#pragma unroll
    for (int b = 0; b < NMAX / 8; ++b) {
      if (live_row<STATIC>(8 * b + 7, k)) {
#pragma unroll
        for (int i = 8 * b; i < 8 * b + 8; ++i) {
          if (live_row<STATIC>(i, k)) {
            h[i] = fmaf(-vv[i], wl, h[i]);
            h[i] = fmaf(-wr[i], vl, h[i]);
          }
        }
      }
    }
  } else {
    // registers are short here: w is read per block, one block ahead
    float wc[8], wn[8];
    load_row<8>(WB, wc);
#pragma unroll
    for (int b = 0; b < NMAX / 8; ++b) {
      if (b + 1 < NMAX / 8) load_row<8>(WB + 8 * b + 8, wn);
      if (live_row<STATIC>(8 * b + 7, k)) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = 8 * b + s;
          h[i] = fmaf(-vv[i], wl, h[i]);
          h[i] = fmaf(-wc[s], vl, h[i]);
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) wc[s] = wn[s];
    }
  }
}

// D with two waves and k a compile-time constant (fully unrolled), step k in
// three barriers.  Thread t's own entry k stands for H[t][k] (H is
// symmetric); the owners of rows k and k + 1 store d_kk and alpha into ad
// before the barrier of the norm's reduction.  v goes through VB, and p
// through WB together with the per-wave partial sums of v^T p (slot 1 of
// red).  Live rows are the aligned 4-row groups past row k, as in tri_step.
// Each slot is rewritten one step later, past a barrier that all its reads
// precede.
template <int NMAX, int NW>
__device__ __forceinline__ void tri_step_static2(float (&h)[NMAX], int k, int t, bool act, float* VB,
                                                 float* WB, float* RS, float* TD, float* TE,
                                                 float* TAU, float* red, float* ad) {
  constexpr int LDN = NMAX + 4;
  const float hk = h[k];
  if (t == k) ad[0] = hk;
  if (t == k + 1) ad[1] = hk;
  const float xn2 = block_reduce<NW>(t > k + 1 ? hk * hk : 0.f, AddOp(), red, 0);
  const float dkk = ad[0], alpha = ad[1];
  float tau = 0.f, beta = alpha, sc = 0.f;
  // a column whose sub-subdiagonal part squares to a subnormal is taken as
  // already reduced (as in tri_step)
  if (xn2 >= kMinNormal) {
    const float nrm = fsqrt(fmaf(alpha, alpha, xn2));
    beta = alpha >= 0.f ? -nrm : nrm;
    tau = (beta - alpha) * frcp(beta);
    sc = frcp(alpha - beta);
  }
  const float vl = (t > k + 1) ? hk * sc : (t == k + 1 ? 1.f : 0.f);
  if (t == 0) {
    TD[k] = dkk;
    TE[k] = beta;
    TAU[k] = tau;
  }
  if (act) VB[t] = vl;
  if (act && t > k) RS[k * LDN + t] = vl;
  __syncthreads();
  float vv[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; i += 4) {
    if (live_row<true>(i + 3, k)) {
      const float4 x4 = *reinterpret_cast<const float4*>(VB + i);
      vv[i] = x4.x; vv[i + 1] = x4.y; vv[i + 2] = x4.z; vv[i + 3] = x4.w;
    } else {
      vv[i] = vv[i + 1] = vv[i + 2] = vv[i + 3] = 0.f;
    }
  }
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; i += 2) {
    if (live_row<true>(i, k)) {
      pa = fmaf(h[i], vv[i], pa);
      pb = fmaf(h[i + 1], vv[i + 1], pb);
    }
  }
  const float pl = (pa + pb) * tau;
  if (act) WB[t] = pl;
  const float part = wave_reduce(pl * vl, AddOp());
  if ((t & 63) == 0) red[NW + (t >> 6)] = part;
  __syncthreads();
  float vp = red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) vp += red[NW + w];
  // w = p + K v with K = -tau/2 v^T p; H <- H - v w^T - w v^T, on this
  // column h - v (w_t + K v_t) - p v_t
  const float K = -0.5f * tau * vp;
  const float wl = fmaf(K, vl, pl);
  const float a = fmaf(K, vl, wl);
#pragma unroll
  for (int i = 0; i < NMAX; i += 4) {
    if (live_row<true>(i + 3, k)) {
      const float4 p4 = *reinterpret_cast<const float4*>(WB + i);
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        h[i + s] = fmaf(-vv[i + s], a, h[i + s]);
        h[i + s] = fmaf(-pv[s], vl, h[i + s]);
      }
    }
  }
}

// ---------------------------------------------------------------------------

template <int NMAX, int RMAX, int DK, int DV_, int FMT>
__global__ __launch_bounds__(64 * ((NMAX + 63) / 64))
__attribute__((amdgpu_waves_per_eu(wave_min_waves<NMAX, RMAX, FMT == kConvert>())))
void compress_wave_kernel(CompressArgs args) {
  const int cap = args.cap, n = args.n, R = args.R;
  float* const __restrict__ U = args.U;
  float* const __restrict__ V = args.V;
  float* const __restrict__ gam = args.gam;
  const int gam_per_row = args.gam_per_row;
  // 16-bit layout: columns 0..R-1 are kept patterns, the fp32 arrays hold
  // columns R..n-1 from their index 0.  It is compiled for R = RMAX only,
  // so that every column's source is known at compile time.  The ring
  // layout's kept columns are fp32 (CompressArgs in seed_launch.h).
  constexpr bool H16 = FMT == kStoreBF16 || FMT == kStoreF16;
  constexpr bool RING = FMT == kStoreRing;
  // the end-of-prefill conversion: H = C C^T of a dense state directly
  // (no factors, no Cholesky), U' = X_R, V' = C^T X_R
  constexpr bool CONV = FMT == kConvert;
  constexpr int KR = H16 ? RMAX : 0;
  using L = Lay<NMAX, RMAX, CONV>;
  constexpr int NW = L::NW, NTH = L::NTH, LDN = L::LDN, LDG = L::LDG;
  constexpr int PARTS = L::PARTS, CH = L::CH, NACT = L::NACT;
  extern __shared__ float4 smem4[];
  float* const sm = reinterpret_cast<float*>(smem4);
  float* const G = sm + L::G;
  float* const RB = sm + L::RB;
  float* const XR = sm + L::XR;
  float* const FA = sm + L::FA;
  float* const FB = sm + L::FB;
  float* const FC = sm + L::FC;
  float* const CB = sm + L::CB;
  float* const VB = sm + L::VB;
  float* const WB = sm + L::WB;
  float* const CB2 = sm + L::CB2;
  float* const TD = sm + L::TD;
  float* const TE = sm + L::TE;
  float* const E2 = sm + L::E2;
  float* const TAU = sm + L::TAU;
  float* const DVs = sm + L::DV;
  float* const IDV = sm + L::IDV;
  float* const IRD = sm + L::IRD;
  float* const BPT = sm + L::BPT;
  int* const BFL = reinterpret_cast<int*>(sm + L::BFL);
  float* const LAM = sm + L::LAM;
  int* const RNK = reinterpret_cast<int*>(sm + L::RNK);
  int* const STA = reinterpret_cast<int*>(sm + L::STA);
  int* const PIV = reinterpret_cast<int*>(sm + L::PIV);
  float* const RED = sm + L::RED;
  // entry i of the staged decay product
  auto gs_at = [=](int i) -> float* {
    if constexpr (L::GS_PAD) return RB + (i >> 2) * LDN + NMAX + (i & 3);
    else return sm + L::GS + i;
  };
  float* const MISC = sm + L::MISC;
  // the Householder reflectors: in the strict upper triangle of R~ (pivot
  // order), or of G for the conversion, which has no R~
  float* const RS = CONV ? G : RB;

  const int t = threadIdx.x;
  const bool act = t < NMAX;
  const size_t ub = args.list != nullptr ? (size_t)args.list[blockIdx.x] : blockIdx.x;
  int kcyc = 0;
  if constexpr (RING) {
    if (ub >= (size_t)args.units_total) return;  // not a unit of this batch
    // the request's latest snapshot, k = A / W, is due while its merge
    // (A = k W + D) has not been reached; else the whole block leaves
    const int A = args.t_snap - args.t_start[ub / args.heads];
    if (A < args.W || A % args.W >= (args.D > 0 ? args.D : 1)) return;
    kcyc = A / args.W;
  }
  float* const Uh = U + ub * cap * DK;
  float* const Vh = V + ub * cap * DV_;
  uint16_t* const Ukh = H16 ? args.Uk + ub * R * DK : nullptr;
  uint16_t* const Vkh = H16 ? args.Vk + ub * R * DV_ : nullptr;
  // ring layout: the kept buffer read and the one written
  const size_t kold = RING ? ((size_t)((kcyc - 1) & 1) * args.units_total + ub) * R : 0;
  const size_t knew = RING ? ((size_t)(kcyc & 1) * args.units_total + ub) * R : 0;
  // fp32 column j of U and V
  auto ucol = [&](int j) -> float* {
    if constexpr (RING)
      return j < R ? args.KU + (kold + j) * DK
                   : Uh + (size_t)(((kcyc - 1) * args.W + j - R) % cap) * DK;
    else
      return Uh + (size_t)(j - KR) * DK;
  };
  auto vcol = [&](int j) -> float* {
    if constexpr (RING)
      return j < R ? args.KV + (kold + j) * DV_
                   : Vh + (size_t)(((kcyc - 1) * args.W + j - R) % cap) * DV_;
    else
      return Vh + (size_t)(j - KR) * DV_;
  };
  // lazily decayed form: U = Diag(gam) U~ (gam per key channel, or one scalar)
  float* const gamh = gam != nullptr ? gam + ub * (gam_per_row ? DK : 1) : nullptr;

  // R~ (with its zero lower part), the eigenvector block and the published
  // vectors start at zero
  if constexpr (!CONV) {
    for (int i = 4 * t; i < NMAX * LDN; i += 4 * NTH)
      *reinterpret_cast<float4*>(RB + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if constexpr (!L::TAIL) {
    // (in G's tail they are written before every read)
    CB[t] = 0.f;
    VB[t] = 0.f;
    WB[t] = 0.f;
  }
  // this column's 1/d and the reciprocal pivot of step t (phase B), kept in
  // registers until phase D stores them for phase H
  float idv_own = 0.f, ird_own = 0.f;
  if (gamh != nullptr) {
    // the decay product of every key row, staged once
    __syncthreads();   // after the zeroing of RB
    for (int i = t; i < DK; i += NTH) *gs_at(i) = gamh[gam_per_row ? i : 0];
    __syncthreads();
  }

  if constexpr (CONV) {
    // @phase A (conversion): the sink a = S vbar / |vbar|^2 (row t of S by
    // thread t), then H = C C^T with C = S - a vbar^T formed on the fly
    float* const vbs = IDV;          // vbar (IDV and IRD: 2 NMAX >= d_v floats)
    float* const asink = DVs;        // a
    const float* const Sh = args.S + ub * DK * DV_;
    for (int e = t; e < DV_; e += NTH) vbs[e] = args.vbar[(size_t)(ub % args.heads) * DV_ + e];
    __syncthreads();
    float nv2 = 0.f;
    for (int e = 0; e < DV_; ++e) nv2 = fmaf(vbs[e], vbs[e], nv2);
    if (act) {
      float p0 = 0.f, p1 = 0.f;
      for (int e = 0; e < DV_; e += 4) {
        const float4 x4 = *reinterpret_cast<const float4*>(Sh + (size_t)t * DV_ + e);
        p0 = fmaf(x4.x, vbs[e], p0);
        p1 = fmaf(x4.y, vbs[e + 1], p1);
        p0 = fmaf(x4.z, vbs[e + 2], p0);
        p1 = fmaf(x4.w, vbs[e + 3], p1);
      }
      const float at = (p0 + p1) / nv2;
      asink[t] = at;
      args.a[ub * DK + t] = at;
    }
    __syncthreads();
    auto scol = [&](int j) -> const float* { return Sh + (size_t)j * DV_; };
    gram<NMAX, NW, DV_, false, kStoreF32, 0, decltype(scol), true>(scol, nullptr, n, G, nullptr,
                                                                   nullptr, false, asink, vbs);
    __syncthreads();
  } else {
    // @phase A: Gram of U and column norms
    gram<NMAX, NW, DK, false, FMT, KR, decltype(ucol), false, false, LDG>(ucol, Ukh, n, G, nullptr,
                                                                         gamh, gam_per_row);
    __syncthreads();
    if (act) {
      // a column whose squared norm is below the normal fp32 range (norm
      // under 1.1e-19: decayed to nothing) is taken as dependent; its
      // reciprocal square root would read the subnormal as zero
      const float gtt = G[t * LDG + t];
      const bool pos = t < n && gtt >= kMinNormal;
      DVs[t] = pos ? fsqrt(gtt) : 0.f;
      idv_own = pos ? frsq(gtt) : 0.f;
    }
    float g[NMAX];
    float dg;   // this column's own diagonal entry of the Schur complement
    {
      const float it = idv_own;
      // the scale d_t^-1 d_i^-1 is one product for both (i, t) and (t, i), so
      // the columns stay exactly symmetric through the Cholesky; 1/d_i is
      // formed from the diagonal as thread i forms its own
  #pragma unroll
      for (int i = 0; i < NMAX; ++i) {
        const float gii = G[i * LDG + i];
        const float di = (i < n && gii >= kMinNormal) ? frsq(gii) : 0.f;
        g[i] = act ? G[i * LDG + t] * (it * di) : 0.f;
      }
      dg = (act && t < n) ? G[t * LDG + t] * (it * it) : 0.f;
    }
    __syncthreads();

    // @phase B: Cholesky with diagonal pivoting of the equilibrated U^T U,
    // thread t owning column t (g) and its own diagonal entry (dg).  Step j
    // takes the unprocessed column p with the largest remaining diagonal
    // (the lowest such t): every multiplier is then at most 1 in size, so
    // a near-dependent column cannot blow the factor up however badly the
    // columns are conditioned.  It stops when that diagonal is at most
    // kPivTol.  Row j of R~ is kept by original column,
    // RB[t LDN + j] = R~[j][t] (0 for the columns taken before), with
    // 1 / R~[j][p] kept by thread j and PIV[j] = p; rows from `kept` on are
    // zero.
    // The pivot value is the reduction's maximum (the pivot's own dg, equal
    // to its column's entry p up to rounding), and row j of R~ is the
    // published column times its reciprocal square root, so a step takes one
    // LDS round trip.  Every thread updates its column with the whole
    // column p: the pivot's own row comes out as zero up to rounding, and
    // the rows of earlier pivots are never read again.
    // (The largest diagonal is reduced at the end of the previous step, so
    // the loop has one exit and its columns are updated in place.)
    bool taken = !(act && t < n && idv_own > 0.f);
    int kept = 0;
    int mypos = -1;   // the step that takes this column as its pivot
    float mx = block_reduce<NW>(taken ? -1.f : dg, MaxOp(), RED, 6);
    for (int j = 0; j < n && mx > kPivTol; ++j) {
      const float cand = taken ? -1.f : dg;
      const int p = block_first<NW>(!taken && cand == mx, RED);
      const float rp = frsq(mx);
      if (t == p) {
        taken = true;
        mypos = j;
  #pragma unroll
        for (int i = 0; i < NMAX; i += 4)
          *reinterpret_cast<float4*>(CB + i) = make_float4(g[i], g[i + 1], g[i + 2], g[i + 3]);
      }
      __syncthreads();
      float wr[NMAX];
      load_row<NMAX>(CB, wr);
      const float ct = CB[t];
      const float r = (act && !taken) ? ct * rp : 0.f;
      if (act) RB[t * LDN + j] = (t == p) ? mx * rp : r;
      if (t == j) ird_own = rp;
      if (t == 0) PIV[j] = p;
      const float rr = r * rp;
  #pragma unroll
      for (int i = 0; i < NMAX; ++i) g[i] = fmaf(-wr[i], rr, g[i]);
      dg = fmaf(-r, r, dg);
      kept = j + 1;
      // the next pivot rewrites CB (one wave reads it in order before that)
      if constexpr (NW > 1) __syncthreads();
      mx = block_reduce<NW>(taken ? -1.f : dg, MaxOp(), RED, 6);
    }
    if (t == 0) MISC[1] = __int_as_float(kept);

    // The pivot order: position j < kept is step j's pivot, the columns
    // never taken follow in column order (0 .. n-1 stay among the first n
    // positions).  PIV[j] is the column at position j, and R~ moves to rows
    // in that order: RB[j LDN + i] = R~[i][PIV[j]], zero for i > j, so R~
    // is lower trapezoidal and the Householder reflectors fit in the strict
    // upper triangle.  The V Gram is formed in the same order, so phases C
    // and H read both as they are.
    {
      const bool rest = act && mypos < 0;
      const unsigned long long b = __ballot(rest);
      int before = __popcll(b & ((1ull << (t & 63)) - 1ull));
      if constexpr (NW > 1) {
        if (t == 0) MISC[2] = __int_as_float(__popcll(b));
        __syncthreads();
        if (t >= 64) before += __float_as_int(MISC[2]);
      }
      if (rest) mypos = kept + before;
    }
    if (act) PIV[mypos] = t;
    __syncthreads();
    {
      float row[NMAX];
      if (act) load_row<NMAX>(RB + t * LDN, row);
      __syncthreads();
      if (act) {
  #pragma unroll
        for (int i = 0; i < NMAX; i += 4)
          *reinterpret_cast<float4*>(RB + mypos * LDN + i) =
              make_float4(row[i], row[i + 1], row[i + 2], row[i + 3]);
      }
    }
    // Gram of V in pivot order, scaled to D V^T V D
    gram<NMAX, NW, DV_, true, FMT, KR, decltype(vcol), false, true, LDG>(
        vcol, Vkh, n, G, DVs, nullptr, false, nullptr, nullptr, PIV);
    __syncthreads();

    // @phase C: Z = R~ G~ in place by column tiles, then H = Z R~^T in place
    // by row tiles (R~ is triangular only in pivot order, so no k-step is
    // skipped)
    {
      constexpr int NT = NMAX / 16;
      const int l = t & 63, w = t >> 6;
      const int ci = l & 15, kk = l >> 4;
  #pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J % NW != w) continue;
        f4v acc[NT];
  #pragma unroll
        for (int I = 0; I < NT; ++I) acc[I] = f4v{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int K = 0; K < NMAX / 4; ++K) {
          const int m = 4 * K + kk;
          const float bv = G[m * LDG + 16 * J + ci];          // G~[m][j]
  #pragma unroll
          for (int I = 0; I < NT; ++I) {
            const float av = RB[m * LDN + 16 * I + ci];        // R~[i][m]
            acc[I] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[I], 0, 0, 0);
          }
        }
  #pragma unroll
        for (int I = 0; I < NT; ++I)
  #pragma unroll
          for (int r = 0; r < 4; ++r) G[(16 * I + 4 * kk + r) * LDG + 16 * J + ci] = acc[I][r];
      }
      __syncthreads();
  #pragma unroll
      for (int I = 0; I < NT; ++I) {
        if (I % NW != w) continue;
        f4v acc[NT];
  #pragma unroll
        for (int J = 0; J < NT; ++J) acc[J] = f4v{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int K = 0; K < NMAX / 4; ++K) {
          const int m = 4 * K + kk;
          const float av = G[(16 * I + ci) * LDG + m];        // Z[i][m]
  #pragma unroll
          for (int J = 0; J < NT; ++J) {
            const float bv = RB[m * LDN + 16 * J + ci];        // R~[j][m]
            acc[J] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[J], 0, 0, 0);
          }
        }
  #pragma unroll
        for (int J = 0; J < NT; ++J)
  #pragma unroll
          for (int r = 0; r < 4; ++r) G[(16 * I + 4 * kk + r) * LDG + 16 * J + ci] = acc[J][r];
      }
      __syncthreads();
    }
  }

  // @phase D: Householder tridiagonalisation, thread t owning column t of H.
  // H is first scaled by the power of two that brings its largest diagonal
  // entry (its largest entry: H is positive semidefinite) into [0.5, 1):
  // exact, the eigenvectors are unchanged and every later stop is relative,
  // and the squares the reflectors form stay clear of the subnormal range,
  // where sqrt and rcp read zero (a content at 1e-6 of a dense state's sink
  // puts H near 1e-12 and its small entries' squares below 1e-38).
  float hs = 1.f;
  {
    const float dg = (act && t < n) ? G[t * LDG + t] : 0.f;
    const float mxd = block_reduce<NW>(dg, MaxOp(), RED, 5);
    if (mxd > 0.f && mxd < 3.0e38f) {
      int ex;
      frexpf(mxd, &ex);
      hs = ldexpf(1.f, -ex);
    }
  }
  float h[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) h[i] = act ? G[i * LDG + t] * hs : 0.f;
  __syncthreads();
  if constexpr (!CONV) {
    // the scales phase H reads: IDV[i] = 1/d_i, IRD[j] = 1/R~[j][PIV[j]]
    // (zero from `kept` on)
    if (act) {
      IDV[t] = idv_own;
      IRD[t] = ird_own;
    }
  }
  if constexpr (NW == 1) {
    // one wave: fully unrolled, so h[k] is a fixed register; H is
    // symmetric, so entry k of this thread's column stands for H[t][k]
#pragma clang loop unroll(full)
    for (int k = 0; k < NMAX - 2; ++k) {
      if (k + 2 < n) {
        const float hk = h[k];
        const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hk), k + 1));
        const float dkk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hk), k));
        tri_step<NMAX, NW, true>(h, k, hk, alpha, dkk, t, act, VB, WB, RS, TD, TE, TAU, RED);
      }
    }
  } else if constexpr (NW == 2 && NMAX <= 96) {
    // two waves (compressions at 64 < n <= 96): fully unrolled as well
#pragma clang loop unroll(full)
    for (int k = 0; k < NMAX - 2; ++k) {
      if (k + 2 < n)
        tri_step_static2<NMAX, NW>(h, k, t, act, VB, WB, RS, TD, TE, TAU, RED, CB);
    }
  } else {
    for (int k = 0; k + 2 < n; ++k) {
      if (t == k) {
#pragma unroll
        for (int i = 0; i < NMAX; i += 4)
          *reinterpret_cast<float4*>(CB + i) = make_float4(h[i], h[i + 1], h[i + 2], h[i + 3]);
      }
      __syncthreads();
      tri_step<NMAX, NW, false>(h, k, CB[t], CB[k + 1], CB[k], t, act, VB, WB, RS, TD, TE, TAU,
                                RED);
    }
  }
  {
    // the trailing 2 x 2 block, from columns n - 1 and n - 2
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
    }
    // pad T to NMAX rows
    if (act && t >= n) TD[t] = kPadDiag;
    if (act && t >= n - 1) TE[t] = 0.f;
    __syncthreads();
    if (act) {
      const float e = t > 0 ? TE[t - 1] : 0.f;
      E2[t] = e * e;
    }
    __syncthreads();
  }

  // @phase E: the R largest eigenvalues of T by multisection
  float tnorm, pivmin;
  {
    float lo_i = 3.0e38f, hi_i = -3.0e38f;
    for (int i = t; i < n; i += NTH) {
      const float rad = fabsf(TE[i]) + (i > 0 ? fabsf(TE[i - 1]) : 0.f);
      lo_i = fminf(lo_i, TD[i] - rad);
      hi_i = fmaxf(hi_i, TD[i] + rad);
    }
    float lo0 = block_reduce<NW>(lo_i, MinOp(), RED, 2);
    float hi0 = block_reduce<NW>(hi_i, MaxOp(), RED, 3);
    tnorm = fmaxf(fabsf(lo0), fabsf(hi0));
    pivmin = tnorm * 1e-30f + 1e-35f;
    lo0 -= 2.f * kEps * tnorm + pivmin;
    hi0 += 2.f * kEps * tnorm + pivmin;
    const int m = NTH / R;                     // threads per eigenvalue (>= 2)
    const int grp = t / m, sub = t - grp * m;
    const bool live = grp < R;
    const int target = n - 1 - grp;            // ascending index of the eigenvalue
    // NP points per thread, NP m per eigenvalue: each pass shrinks the
    // interval NP m + 1 times.  The Sturm count's reciprocal is a
    // quarter-rate instruction, and with two units per SIMD the issue rate
    // bounds the kernel: one point per thread does the least work per
    // decade (NP / log(NP m + 1)), 5 % faster at n = 48 than two.
    // A shift seeds inverse iteration, whose vector for lam_c picks up
    // lam_{c+1}'s in the ratio (shift error) / (lam_c - lam_{c+1}) per
    // solve.  The spectrum is graded (pivoted R~ puts the large rows first),
    // and its leading R eigenvalues can reach far below eps |T|: a dense
    // state's n = d_k Gram, or a window whose keys decay to nothing in some
    // channels, where lam_R is 1e-9 |T|.  The stop is therefore relative to
    // the eigenvalue, floored at kEigFloor eps |T| (a direction of content
    // below sqrt(kEigFloor eps) of the largest one).  An absolute stop at a
    // few eps |T| put such a shift above its eigenvalue by orders of
    // magnitude, and lost about sqrt(eps) of the content.
    constexpr int NP = 1;
    const float frac = 1.f / (float)(NP * m + 1);
    const float tol_rel = 2.f * kEps;
    const float tol_floor = kEigFloor * kEps * tnorm + pivmin;
    // up to 64 rows, T sits in registers (padded rows never count)
    constexpr bool TREG = NMAX <= 64;
    float dr[TREG ? NMAX : 4], er[TREG ? NMAX : 4];
    if constexpr (TREG) {
      load_row<NMAX>(TD, dr);
      load_row<NMAX>(E2, er);
    }
    float lo = lo0, hi = hi0;
    for (int it = 0; it < 48; ++it) {
      const bool done = !live || (hi - lo) <= tol_rel * (fabsf(lo) + fabsf(hi)) + tol_floor;
      if (block_all<NW>(done, RED, 4)) break;
      const float step = (hi - lo) * frac;
      float x[NP], qv[NP];
      int cnt[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        x[p] = lo + step * (float)(NP * sub + p + 1);
        qv[p] = 1.f;
        cnt[p] = 0;
      }
      if constexpr (TREG) {
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            float q = (dr[i] - x[p]) - er[i] * frcp(qv[p]);
            q = fabsf(q) < pivmin ? -pivmin : q;
            cnt[p] += q < 0.f;
            qv[p] = q;
          }
        }
      } else {
        for (int i4 = 0; i4 < n; i4 += 4) {
          float dd[4], ee[4];
          load_row<4>(TD + i4, dd);
          load_row<4>(E2 + i4, ee);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              float q = (dd[s] - x[p]) - ee[s] * frcp(qv[p]);
              q = fabsf(q) < pivmin ? -pivmin : q;
              cnt[p] += q < 0.f;
              qv[p] = q;
            }
          }
        }
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        BPT[NP * t + p] = x[p];
        BFL[NP * t + p] = cnt[p] > target;
      }
      __syncthreads();
      if (live && !done) {
        for (int s2 = 0; s2 < NP * m; ++s2) {
          const float ps = BPT[NP * grp * m + s2];
          if (BFL[NP * grp * m + s2]) hi = fminf(hi, ps);
          else lo = fmaxf(lo, ps);
        }
      }
      __syncthreads();
    }
    if (live && sub == 0) LAM[grp] = 0.5f * (lo + hi);
  }
  __syncthreads();

  // @phase F: eigenvectors of T by inverse iteration (the eigenvector block
  // starts at zero; it shares LDS with G, or the bisection points, before)
  for (int i = 4 * t; i < NMAX * RMAX; i += 4 * NTH)
    *reinterpret_cast<float4*>(XR + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  if (t < 64) {
    // separate equal shifts: lam'_c = min_{j <= c} (lam_j - (c - j) sep_j),
    // sep_j = 10 eps |lam_j| (floored as the bisection's stop).  A
    // separation scaled by |T| would move a small shift by more than the
    // gap to its neighbour and mix their vectors.
    float lc = 3.0e38f;
    for (int j = 0; j < R; ++j)
      if (j <= t) {
        const float sep = 10.f * kEps * fabsf(LAM[j]) + kEigFloor * kEps * tnorm;
        lc = fminf(lc, LAM[j] - (float)(t - j) * sep);
      }
    // runs of close eigenvalues: the vector of c is computed in round
    // c - (first index of its run)
    const float prev = __shfl_up(lc, 1);
    const bool head = t == 0 || !(prev - lc < kClusterTol * tnorm);
    const unsigned long long heads = __ballot(head && t < R);
    const unsigned long long upto = heads & ((t >= 63) ? ~0ull : ((2ull << t) - 1ull));
    const int start = upto ? 63 - __clzll(upto) : 0;
    const int rk = t - start;
    const float maxr = wave_reduce(t < R ? (float)rk : 0.f, MaxOp());
    if (t < R) {
      LAM[t] = lc;
      RNK[t] = rk;
      STA[t] = start;
    }
    if (t == 0) MISC[0] = maxr;
  }
  __syncthreads();
  {
    const int maxr = (int)MISC[0];
    const float tiny = kEps * tnorm + 1e-30f;
    const int c = t;
    // T is read from LDS (the same entry in every lane, independent of the
    // serial chain, so the unrolled loops issue the reads early); one wave
    // keeps the two superdiagonals of U in registers, two waves in LDS
    constexpr bool FREG = L::FREG;
    for (int rnd = 0; rnd <= maxr; ++rnd) {
      if (c < R && RNK[c] == rnd) {
        const float lc = LAM[c];
        float x[NMAX];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c) : 0.f;
        for (int it = 0; it < kInvIters; ++it) {
          // factor T - lc I with partial pivoting while eliminating x; the
          // reciprocal pivots go to LDS, the two superdiagonals of U to
          // registers (one wave) or LDS, the eliminated right-hand side
          // stays in x
          float fb[FREG ? NMAX : 1], fc[FREG ? NMAX : 1];
          float a = TD[0] - lc, b1 = TE[0], b2 = 0.f, rr = x[0];
#pragma unroll
          for (int i = 0; i + 1 < NMAX; ++i) {
            const float lw = TE[i];
            const float ap = TD[i + 1] - lc;
            const float b1p = (i + 2 < NMAX) ? TE[i + 1] : 0.f;
            const float rp = x[i + 1];
            const bool sw = fabsf(lw) > fabsf(a);
            const float pa = sw ? lw : ((a != 0.f) ? a : tiny);
            const float ipa = frcp(pa);
            FA[i * RMAX + c] = ipa;
            if constexpr (FREG) {
              fb[i] = sw ? ap : b1;
              fc[i] = sw ? b1p : b2;
            } else {
              FB[i * RMAX + c] = sw ? ap : b1;
              FC[i * RMAX + c] = sw ? b1p : b2;
            }
            x[i] = sw ? rp : rr;
            const float mm = (sw ? a : lw) * ipa;
            const float na = fmaf(-mm, sw ? ap : b1, sw ? b1 : ap);
            const float nb1 = fmaf(-mm, sw ? b1p : b2, sw ? b2 : b1p);
            const float nr = fmaf(-mm, sw ? rp : rr, sw ? rr : rp);
            a = na; b1 = nb1; b2 = 0.f; rr = nr;
          }
          FA[(NMAX - 1) * RMAX + c] = frcp((a != 0.f) ? a : tiny);
          if constexpr (FREG) {
            fb[NMAX - 1] = 0.f;
            fc[NMAX - 1] = 0.f;
          } else {
            FB[(NMAX - 1) * RMAX + c] = 0.f;
            FC[(NMAX - 1) * RMAX + c] = 0.f;
          }
          x[NMAX - 1] = rr;
          // mx is the largest |x_i|; fmaxf drops NaN, so an overflow that
          // turned into inf - inf or 0 inf is caught by fin
          float x1 = 0.f, x2 = 0.f, mx = 0.f;
          bool fin = true;
#pragma unroll
          for (int i = NMAX - 1; i >= 0; --i) {
            float ub1, ub2;
            if constexpr (FREG) {
              ub1 = fb[i];
              ub2 = fc[i];
            } else {
              ub1 = FB[i * RMAX + c];
              ub2 = FC[i * RMAX + c];
            }
            const float xi = (x[i] - ub1 * x1 - ub2 * x2) * FA[i * RMAX + c];
            x[i] = xi;
            mx = fmaxf(mx, fabsf(xi));
            fin = fin && fabsf(xi) < 3.0e38f;
            x2 = x1;
            x1 = xi;
          }
          if (!fin || !(mx > 0.f)) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c + 7 * it + 1) : 0.f;
            continue;
          }
          const float imx = frcp(mx);
#pragma unroll
          for (int i = 0; i < NMAX; ++i) x[i] *= imx;
          for (int pass = 0; pass < 2; ++pass) {
            for (int j = STA[c]; j < c; ++j) {
              float dt = 0.f;
#pragma unroll
              for (int i = 0; i < NMAX; ++i) dt = fmaf(x[i], XR[i * RMAX + j], dt);
#pragma unroll
              for (int i = 0; i < NMAX; ++i) x[i] = fmaf(-dt, XR[i * RMAX + j], x[i]);
            }
          }
          float nx = 0.f;
#pragma unroll
          for (int i = 0; i < NMAX; ++i) nx = fmaf(x[i], x[i], nx);
          if (nx > 0.f) {
            const float inx = frsq(nx);
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] *= inx;
          } else {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c + 7 * it + 3) : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < NMAX; ++i) XR[i * RMAX + c] = x[i];
      }
      __syncthreads();
    }
  }

  // one modified Gram-Schmidt pass over the R vectors; thread (c, part)
  // holds rows part * CH .. part * CH + CH - 1 of vector c
  const int c = t / PARTS, part = t % PARTS;
  const bool w0 = t < NACT;
  float y[CH];
#pragma unroll
  for (int s = 0; s < CH; ++s) y[s] = (w0 && c < R) ? XR[(part * CH + s) * RMAX + c] : 0.f;
  for (int c0 = 0; c0 < R; ++c0) {
    float* const buf = CB2 + (c0 & 1) * NMAX;
    if (w0 && c == c0) {
#pragma unroll
      for (int s = 0; s < CH; ++s) buf[part * CH + s] = y[s];
    }
    __syncthreads();
    if (w0) {
      float nrm2 = 0.f, dt = 0.f;
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const float xb = buf[part * CH + s];
        nrm2 = fmaf(xb, xb, nrm2);
        dt = fmaf(y[s], xb, dt);
      }
      nrm2 = group_sum<PARTS>(nrm2);
      dt = group_sum<PARTS>(dt);
      const float f = (c > c0 && c < R && nrm2 > 0.f) ? dt * frcp(nrm2) : 0.f;
      const float sc = (c == c0) ? (nrm2 > 0.f ? frsq(nrm2) : 0.f) : 1.f;
#pragma unroll
      for (int s = 0; s < CH; ++s) y[s] = fmaf(-f, buf[part * CH + s], y[s]) * sc;
    }
  }

  // @phase G: back-transform Y -> Q Y through the reflectors (rows of RS,
  // entries > k; the entries <= k of row k hold R~ and read as zero)
  if (w0) {
    // reflector k (this lane's rows) and tau_k are read one step ahead; the
    // loop runs over every k < NMAX - 2 so that it unrolls, and skips
    // k > n - 3
    float vk[CH], vn[CH];
    load_row<CH>(RS + (NMAX - 3) * LDN + part * CH, vk);
    float tk = TAU[NMAX - 3], tn = 0.f;
#pragma unroll
    for (int k = NMAX - 3; k >= 0; --k) {
      if (k > 0) {
        load_row<CH>(RS + (k - 1) * LDN + part * CH, vn);
        tn = TAU[k - 1];
      }
#pragma unroll
      for (int s = 0; s < CH; ++s) vk[s] = (part * CH + s > k) ? vk[s] : 0.f;
      if (k <= n - 3) {
        float pd0 = 0.f, pd1 = 0.f;
#pragma unroll
        for (int s = 0; s < CH; s += 2) {
          pd0 = fmaf(vk[s], y[s], pd0);
          pd1 = fmaf(vk[s + 1], y[s + 1], pd1);
        }
        const float pd = group_sum<PARTS>(pd0 + pd1) * tk;
#pragma unroll
        for (int s = 0; s < CH; ++s) y[s] = fmaf(-pd, vk[s], y[s]);
      }
#pragma unroll
      for (int s = 0; s < CH; ++s) vk[s] = vn[s];
      tk = tn;
    }
#pragma unroll
    for (int s = 0; s < CH; ++s) XR[(part * CH + s) * RMAX + c] = y[s];
  }
  __syncthreads();

  if constexpr (!CONV) {
    // @phase H: P2 = D R~^T X_R (MFMA, into FA), then T' = D^-1 R~^-1 X_R;
    // both by original column (row PIV[p] for R~'s row p in pivot order)
    {
      constexpr int NT = NMAX / 16;
      const int l = t & 63, w = t >> 6;
      const int ci = l & 15, kk = l >> 4;
  #pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J % NW != w) continue;
  #pragma unroll
        for (int C = 0; C < RMAX / 16; ++C) {
          f4v acc = f4v{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int K = 0; K < NMAX / 4; ++K) {
            // R~[i][PIV[p]] for p = 16 J + ci, i = 4 K + kk; beyond i = p the
            // row holds a reflector
            const float av = (4 * K + kk <= 16 * J + ci) ? RB[(16 * J + ci) * LDN + 4 * K + kk]
                                                         : 0.f;
            const float bv = XR[(4 * K + kk) * RMAX + 16 * C + ci];  // X_R[i][c]
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
          }
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = PIV[16 * J + 4 * kk + r];
            FA[j * RMAX + 16 * C + ci] = DVs[j] * acc[r];
          }
        }
      }
    }
    __syncthreads();
    // the rows of T' that no step reaches (dropped columns) stay zero; y
    // holds X_R in registers
    for (int i = 4 * t; i < NMAX * RMAX; i += 4 * NTH)
      *reinterpret_cast<float4*>(XR + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    if (w0) {
      // R11 y = X_R with R11[m][l] = R~[m][PIV[l]] = RB[l LDN + m], upper
      // triangular, from the last kept step up: the lane owning row i
      // broadcasts t_i to its group and stores t_i / d_p as row p = PIV[i]
      // of T'.  The reciprocal pivots of the lane's own rows are read before
      // the serial chain, and row i of RB one step ahead.  Its entries
      // m > i (a reflector) only reach rows of y already solved.
      const int kept = __float_as_int(MISC[1]);
      float ird[CH];
  #pragma unroll
      for (int s = 0; s < CH; ++s) ird[s] = IRD[part * CH + s];
      float rc[CH], rn[CH];
  #pragma unroll
      for (int s = 0; s < CH; ++s) rc[s] = RB[(NMAX - 1) * LDN + part * CH + s];
  #pragma unroll
      for (int i = NMAX - 1; i >= 0; --i) {
        if (i > 0) {
  #pragma unroll
          for (int s = 0; s < CH; ++s) rn[s] = RB[(i - 1) * LDN + part * CH + s];   // R~[m][PIV[i-1]]
        }
        if (i < kept) {
          const int own = i / CH, si = i - (i / CH) * CH;
          const float yi = y[si] * ird[si];
          float ti = (part == own) ? yi : 0.f;
          switch (own) {
            case 0: ti = group_bcast<PARTS, 0>(ti); break;
            case 1: ti = group_bcast<PARTS, 1>(ti); break;
            case 2: if constexpr (PARTS > 2) ti = group_bcast<PARTS, 2>(ti); break;
            default: if constexpr (PARTS > 3) ti = group_bcast<PARTS, 3>(ti); break;
          }
          const int pi = PIV[i];
          if (part == own && c < R) XR[pi * RMAX + c] = ti * IDV[pi];
  #pragma unroll
          for (int s = 0; s < CH; ++s) y[s] = fmaf(-rc[s], ti, y[s]);
        }
  #pragma unroll
        for (int s = 0; s < CH; ++s) rc[s] = rn[s];
      }
    }
    __syncthreads();
  }

  if constexpr (CONV) {
    // @phase I (conversion): U' = X_R; V' = C^T X_R = S^T X_R - vbar beta^T
    // with beta = X_R^T a, by MFMA over 16-row tiles of V'
    const float* const Sh = args.S + ub * DK * DV_;
    const float* const vbs = IDV;
    const float* const asink = DVs;
    float* const beta_s = LAM;       // the eigenvalues are not needed any more
    for (int i = t; i < NMAX * RMAX; i += NTH) {
      const int row = i / RMAX, c = i - (i / RMAX) * RMAX;
      if (c < R) Uh[(size_t)c * DK + row] = XR[row * RMAX + c];
    }
    if (t < RMAX) {
      float b = 0.f;
      for (int j = 0; j < NMAX; ++j) b = fmaf(asink[j], XR[j * RMAX + t], b);
      beta_s[t] = b;
    }
    __syncthreads();
    constexpr int NK = NMAX / 4, NC = RMAX / 16, TV = DV_ / 16;
    const int l = t & 63, w = t >> 6;
    const int ci = l & 15, kk = l >> 4;
    float bx[NC][NK];
#pragma unroll
    for (int C = 0; C < NC; ++C)
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const int cc = 16 * C + ci;
        bx[C][K] = cc < R ? XR[(4 * K + kk) * RMAX + cc] : 0.f;
      }
    for (int E = w; E < TV; E += NW) {
      f4v acc[NC];
#pragma unroll
      for (int C = 0; C < NC; ++C) acc[C] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const float av = Sh[(size_t)(4 * K + kk) * DV_ + 16 * E + ci];     // S[j][e]
#pragma unroll
        for (int C = 0; C < NC; ++C)
          acc[C] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bx[C][K], acc[C], 0, 0, 0);
      }
#pragma unroll
      for (int C = 0; C < NC; ++C) {
        const int cc = 16 * C + ci;
        if (cc < R) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 16 * E + 4 * kk + r;
            Vh[(size_t)cc * DV_ + e] = fmaf(-vbs[e], beta_s[cc], acc[C][r]);
          }
        }
      }
    }
  } else {
    // @phase I: U' = U T' and V' = V P2, MFMA over 16-row tiles, written in
    // place.  A tile reads and writes only its own rows; the next tile's rows
    // are loaded before the current tile is computed.
    {
      constexpr int NK = NMAX / 4, NC = RMAX / 16;
      constexpr int TU = DK / 16, TT = DK / 16 + DV_ / 16;
      static_assert(TU % NW == 0 && TT % NW == 0, "row tiles per wave");
      const int l = t & 63, w = t >> 6;
      const int ci = l & 15, kk = l >> 4;
      float bt[NC][NK], bp[NC][NK];
  #pragma unroll
      for (int C = 0; C < NC; ++C)
  #pragma unroll
        for (int K = 0; K < NK; ++K) {
          const int j = 4 * K + kk, cc = 16 * C + ci;
          const bool ok = j < n && cc < R;
          bt[C][K] = ok ? XR[j * RMAX + cc] : 0.f;
          bp[C][K] = ok ? FA[j * RMAX + cc] : 0.f;
        }
      float av[NK], an[NK];
      // in the lazy form, row 16 E + ci of U carries its decay factor: one
      // scale per U tile of this wave, read before the tile pipeline
      float rsc[TU / NW];
  #pragma unroll
      for (int q = 0; q < TU / NW; ++q) rsc[q] = 1.f;
      if (gamh != nullptr) {
  #pragma unroll
        for (int q = 0; q < TU / NW; ++q) rsc[q] = *gs_at(16 * (q * NW + w) + ci);
      }
      // wave w takes tiles E = q NW + w; the U tiles come first and TU is a
      // multiple of NW, so whether tile q is a U tile does not depend on w
      auto load_tile = [&](int q, float (&dst)[NK]) {
        const bool isu = q < TU / NW;
        const int E = q * NW + w;
        const int ld = isu ? DK : DV_;
        const int row = isu ? 16 * E : 16 * (E - TU);
        if constexpr (!H16) {
  #pragma unroll
          for (int K = 0; K < NK; ++K) {
            const int j = 4 * K + kk;
            dst[K] = (j < n) ? (isu ? ucol(j) : vcol(j))[row + ci] : 0.f;
          }
        } else {
          const float* base = isu ? Uh + 16 * E : Vh + 16 * (E - TU);
          const uint16_t* basek = isu ? Ukh + 16 * E : Vkh + 16 * (E - TU);
  #pragma unroll
          for (int K = 0; K < NK; ++K) {
            const int j = 4 * K + kk;
            float x = 0.f;
            if (j < KR) x = widen16<FMT>(basek[(size_t)j * ld + ci]);
            else if (j < n) x = base[(size_t)(j - KR) * ld + ci];
            dst[K] = x;
          }
        }
        if (isu) {
  #pragma unroll
          for (int K = 0; K < NK; ++K) dst[K] *= rsc[q < TU / NW ? q : 0];
        }
      };
      load_tile(0, av);
  #pragma unroll
      for (int q = 0; q < TT / NW; ++q) {
        if (q + 1 < TT / NW) load_tile(q + 1, an);
        const bool isu = q < TU / NW;
        const int E = q * NW + w;
        f4v acc[NC];
  #pragma unroll
        for (int C = 0; C < NC; ++C) acc[C] = f4v{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int K = 0; K < NK; ++K)
  #pragma unroll
          for (int C = 0; C < NC; ++C)
            acc[C] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[K], isu ? bt[C][K] : bp[C][K], acc[C],
                                                          0, 0, 0);
        const int ld = isu ? DK : DV_;
        if constexpr (RING) {
          // U~' = Diag(1 / gam) U' (the decay product at the snapshot keeps
          // running), into the other kept buffer
          float* base = isu ? args.KU + knew * DK + 16 * E : args.KV + knew * DV_ + 16 * (E - TU);
          float sc[4] = {1.f, 1.f, 1.f, 1.f};
          if (isu) {
  #pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = 1.f / *gs_at(16 * E + 4 * kk + i);
          }
  #pragma unroll
          for (int C = 0; C < NC; ++C) {
            const int cc = 16 * C + ci;
            if (cc < R)
              *reinterpret_cast<float4*>(base + (size_t)cc * ld + 4 * kk) =
                  make_float4(acc[C][0] * sc[0], acc[C][1] * sc[1], acc[C][2] * sc[2],
                              acc[C][3] * sc[3]);
          }
        } else if constexpr (FMT == kStoreF32) {
          float* base = isu ? Uh + 16 * E : Vh + 16 * (E - TU);
  #pragma unroll
          for (int C = 0; C < NC; ++C) {
            const int cc = 16 * C + ci;
            if (cc < R)
              *reinterpret_cast<float4*>(base + (size_t)cc * ld + 4 * kk) =
                  make_float4(acc[C][0], acc[C][1], acc[C][2], acc[C][3]);
          }
        } else {
          // rows 16 E' + 4 kk .. + 3 of column cc: one group of four elements
          // of the unit's factor block (U column cc at f = cc d_k + row, V
          // column cc at f = R d_k + cc d_v + row)
          uint16_t* basek = isu ? Ukh + 16 * E : Vkh + 16 * (E - TU);
          const uint32_t fb = isu ? 16u * E + 4u * kk : (uint32_t)R * DK + 16u * (E - TU) + 4u * kk;
  #pragma unroll
          for (int C = 0; C < NC; ++C) {
            const int cc = 16 * C + ci;
            if (cc < R) {
              const float xv[4] = {acc[C][0], acc[C][1], acc[C][2], acc[C][3]};
              *reinterpret_cast<uint2*>(basek + (size_t)cc * ld + 4 * kk) =
                  round_pack4<FMT>(xv, args.stochastic != 0, fb + (uint32_t)(cc * ld),
                                   (uint32_t)ub, args.epoch, args.key_lo, args.key_hi);
            }
          }
        }
  #pragma unroll
        for (int K = 0; K < NK; ++K) av[K] = an[K];
      }
    }
  }
  if (gamh != nullptr && !RING) {
    // U' is stored at true scale: the decay product starts again from 1
    __syncthreads();
    if (gam_per_row) {
      for (int i = t; i < DK; i += NTH) gamh[i] = 1.f;
    } else if (t == 0) {
      gamh[0] = 1.f;
    }
  }
}

template <int NMAX, int RMAX, bool NO_RB = false>
constexpr size_t wave_lds_bytes() {
  return 4 * (size_t)Lay<NMAX, RMAX, NO_RB>::TOTAL;
}

template <int NMAX, int RMAX, int DK, int DV_, int FMT>
hipError_t wave_go(const CompressArgs& args, hipStream_t s) {
  constexpr size_t bytes = wave_lds_bytes<NMAX, RMAX, FMT == kConvert>();
  // the LDS limit is raised once per device, so that later calls (also
  // under stream capture) only enqueue the kernel
  static std::atomic<unsigned long long> lds_set{0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(lds_set.load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(compress_wave_kernel<NMAX, RMAX, DK, DV_, FMT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (err != hipSuccess) return err;
    lds_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((compress_wave_kernel<NMAX, RMAX, DK, DV_, FMT>), dim3(args.units),
                     dim3(Lay<NMAX, RMAX, FMT == kConvert>::NTH), bytes, s, args);
  return hipGetLastError();
}

// NMAX: n rounded up to a multiple of 16; RMAX: R rounded up to 16 or 32.
inline int wave_nmax(int n) { return (n + 15) / 16 * 16; }

inline size_t wave_lds_bytes_for(int n, int R) {
  const int nm = wave_nmax(n);
  const bool r16 = R <= 16;
  switch (nm) {
    case 16: return wave_lds_bytes<16, 16>();
    case 32: return r16 ? wave_lds_bytes<32, 16>() : wave_lds_bytes<32, 32>();
    case 48: return r16 ? wave_lds_bytes<48, 16>() : wave_lds_bytes<48, 32>();
    case 64: return r16 ? wave_lds_bytes<64, 16>() : wave_lds_bytes<64, 32>();
    case 80: return r16 ? wave_lds_bytes<80, 16>() : wave_lds_bytes<80, 32>();
    default: return r16 ? wave_lds_bytes<96, 16>() : wave_lds_bytes<96, 32>();
  }
}

template <int DK, int DV_, int FMT>
hipError_t wave_dispatch(const CompressArgs& a, hipStream_t s) {
  const int nm = wave_nmax(a.n);
  // the 16-bit layout is compiled for R = RMAX
  if (FMT != kStoreF32 && a.R != 16 && a.R != 32) return hipErrorInvalidValue;
  if (a.R <= 16) {
    switch (nm) {
      case 16: return wave_go<16, 16, DK, DV_, FMT>(a, s);
      case 32: return wave_go<32, 16, DK, DV_, FMT>(a, s);
      case 48: return wave_go<48, 16, DK, DV_, FMT>(a, s);
      case 64: return wave_go<64, 16, DK, DV_, FMT>(a, s);
      case 80: return wave_go<80, 16, DK, DV_, FMT>(a, s);
      case 96: return wave_go<96, 16, DK, DV_, FMT>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nm) {
    case 32: return wave_go<32, 32, DK, DV_, FMT>(a, s);
    case 48: return wave_go<48, 32, DK, DV_, FMT>(a, s);
    case 64: return wave_go<64, 32, DK, DV_, FMT>(a, s);
    case 80: return wave_go<80, 32, DK, DV_, FMT>(a, s);
    case 96: return wave_go<96, 32, DK, DV_, FMT>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// The conversion: n = d_k columns (NMAX = d_k), RMAX from R.
template <int DK, int DV_>
hipError_t convert_dispatch(const CompressArgs& a, hipStream_t s) {
  if (a.n != DK) return hipErrorInvalidValue;
  if (a.R <= 16) return wave_go<DK, 16, DK, DV_, kConvert>(a, s);
  if (a.R <= 32) return wave_go<DK, 32, DK, DV_, kConvert>(a, s);
  return hipErrorInvalidValue;
}

inline size_t convert_lds_bytes_for(int d_k, int R) {
  const bool r16 = R <= 16;
  if (d_k == 128) return r16 ? wave_lds_bytes<128, 16, true>() : wave_lds_bytes<128, 32, true>();
  return r16 ? wave_lds_bytes<64, 16, true>() : wave_lds_bytes<64, 32, true>();
}

}  // namespace wave
}  // namespace seed
