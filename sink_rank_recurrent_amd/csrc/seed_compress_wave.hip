// Compression of the factors to rank R with one wave64 per (request, head).
//
// Same mathematics as the workgroup kernel in seed_compress.hip (the best
// rank-R approximation of the content U V^T, the sink untouched; SEED
// figures and tables on thelatestinai.com, Fig. 1 (b) caption), computed
// through the top-R eigenvectors of the n x n core
//     H = R_U (V^T V) R_U^T,   U^T U = R_U^T R_U   (n = R + W <= 64),
// but with a direct symmetric eigensolver instead of Jacobi sweeps:
//   A  Gram matrices U^T U and V^T V with v_mfma_f32_16x16x4f32;
//   B  column-equilibrated Cholesky of U^T U, lane l owning column l;
//   C  H column by column (lane l: H e_l = R (G~ r_l), r_l = row l of R);
//   D  Householder reduction of H to tridiagonal T (lane l owns column l);
//   E  the R + 1 largest eigenvalues of T by multisection on Sturm counts,
//      all 64 lanes splitting each interval;
//   F  their eigenvectors by inverse iteration with a pivoted tridiagonal
//      solve, re-orthogonalised (twice) inside clusters of close
//      eigenvalues, clusters handled in successive rounds;
//   G  back-transform through the Householder reflectors (X_R = Q Y);
//   H  P2 = D R^T X_R and T' = D^-1 R^-1 X_R;
//   I  U' = U T' and V' = V P2, each lane owning rows of U and V.
// A workgroup is a single wave, so the workgroup barriers below order LDS
// traffic inside the wave and never wait for other waves.
#include "seed_device.h"
#include "seed_launch.h"

namespace seed {

namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kEps = 1.1920928955078125e-7f;   // 2^-23
constexpr float kPivTol = 1e-5f;                   // dependent-column threshold (relative)
// Shifts closer than kClusterTol |T| are re-orthogonalised during inverse
// iteration (their vectors could otherwise come out nearly parallel); all
// top-R vectors then go through one modified Gram-Schmidt pass.
constexpr float kClusterTol = 1e-5f;
constexpr int kInvIters = 2;
// T is padded to NMAX rows with this diagonal and zero couplings: the padded
// eigenvalues are never among the counted ones and the padded entries of
// every solve are exactly 0, so the loops below need no bounds tests.
constexpr float kPadDiag = 1.0e30f;

// Sum / min / max over the 64 lanes, returned to every lane.  Inside each
// row of 16 lanes: DPP butterflies (xor 1, xor 2, mirror within 8, mirror
// within 16); across the 4 rows: one readlane per row.
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
__device__ __forceinline__ float wave_sum(float x) { return wave_reduce(x, AddOp()); }
__device__ __forceinline__ float wave_min(float x) { return wave_reduce(x, MinOp()); }
__device__ __forceinline__ float wave_max(float x) { return wave_reduce(x, MaxOp()); }
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// a[idx] for a wave-uniform runtime idx without dynamic register indexing
// (which would put the array in scratch memory).
template <int N>
__device__ __forceinline__ float pick(const float (&a)[N], int idx) {
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) r = (i == idx) ? a[i] : r;
  return r;
}

// Deterministic start vector of inverse iteration, entries in [0.5, 1.5).
__device__ __forceinline__ float start_entry(int i, int c) {
  uint32_t h = (uint32_t)(i + 1) * 2654435761u ^ (uint32_t)(c + 1) * 2246822519u;
  h ^= h >> 13;
  h *= 3266489917u;
  h ^= h >> 16;
  return (float)(h & 0xFFFFu) * (1.0f / 65536.0f) + 0.5f;
}

template <int NMAX>
struct WaveLds {
  static constexpr int LDN = NMAX + 1;
  float* G;     // [NMAX][LDN] Gram staging, then G~_V, then Householder vectors (row k)
  float* Rb;    // [NMAX][LDN] R, column-major: Rb[m * LDN + i] = R[i][m]
  float* XR;    // [NMAX][R]   eigenvectors, then T'
  float4* F;    // NMAX * max(R, 16) float4: per-lane z staging [NMAX][64] (phase C),
                //   inverse-iteration factors [NMAX][R] (F), P2 [NMAX][R] floats (H, I)
  float* vb;    // [NMAX]
  float* wb;    // [NMAX]
  float* td;    // [NMAX] diagonal of T
  float* te;    // [NMAX] off-diagonal of T
  float* tau;   // [NMAX]
  float* dv;    // [NMAX] column norms of U
  float* bpt;   // [64]
  int* bfl;     // [64]
  float* lam;   // [36]
  int* rnk;     // [36]
  float* misc;  // [4]
  float* cb;    // [NMAX] one lane's column, broadcast to the others
};

__host__ __device__ inline size_t wave_f_floats(int nmax, int R) {
  return 4 * (size_t)nmax * (R > 16 ? R : 16);
}

__host__ __device__ inline size_t wave_lds_floats(int nmax, int R) {
  const size_t ldn = nmax + 1;
  return 2 * nmax * ldn + (size_t)nmax * R + wave_f_floats(nmax, R) + 6 * (size_t)nmax + 64 + 64 +
         36 + 36 + 4 + (size_t)nmax;
}

template <int NMAX>
__device__ inline WaveLds<NMAX> wave_carve(float* base, int R) {
  constexpr int LDN = NMAX + 1;
  WaveLds<NMAX> L;
  float* p = base;
  L.G = p; p += NMAX * LDN;
  L.Rb = p; p += NMAX * LDN;
  L.XR = p; p += NMAX * R;
  L.F = reinterpret_cast<float4*>(p); p += wave_f_floats(NMAX, R);   // offset: multiple of 4 floats
  L.vb = p; p += NMAX;
  L.wb = p; p += NMAX;
  L.td = p; p += NMAX;
  L.te = p; p += NMAX;
  L.tau = p; p += NMAX;
  L.dv = p; p += NMAX;
  L.bpt = p; p += 64;
  L.bfl = reinterpret_cast<int*>(p); p += 64;
  L.lam = p; p += 36;
  L.rnk = reinterpret_cast<int*>(p); p += 36;
  L.misc = p; p += 4;
  L.cb = p;
  return L;
}

// A: G[i][j] = sum_e X_i[e] X_j[e] for i, j < NMAX (zero outside n), X_j the
// columns of one unit's factor (D entries each).  MFMA 16x16x4: lane l
// feeds column (tile*16 + l%16) and the entries of k-slot l/16; the k
// index runs over e = (l/16) * D/4 + s, the same for both operands.
template <int NMAX, int D>
__device__ __forceinline__ void gram_mfma(const float* __restrict__ X, int n, float* G) {
  constexpr int LDN = NMAX + 1;
  constexpr int NT = NMAX / 16;
  constexpr int NP = NT * (NT + 1) / 2;
  constexpr int KPL = D / 4;
  constexpr int KC = 16;
  const int l = threadIdx.x;
  const int ci = l & 15, kk = l >> 4;
  f4v acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < KPL; s0 += KC) {
    float x[NT][KC];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = t * 16 + ci;
      if (col < n) {
        const float* src = X + (size_t)col * D + kk * KPL + s0;
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
  // lane l holds D[4 * (l/16) + r][l % 16] of each 16 x 16 tile
  int p = 0;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = I; J < NT; ++J) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + 4 * kk + r, j = J * 16 + ci;
        G[i * LDN + j] = acc[p][r];
        G[j * LDN + i] = acc[p][r];
      }
      ++p;
    }
}

template <int NMAX, int DK, int DV, int RMAX>
__global__ __launch_bounds__(64) void compress_wave_kernel(float* __restrict__ U,
                                                          float* __restrict__ V, int cap, int n,
                                                          int R) {
  extern __shared__ float smem[];
  constexpr int LDN = NMAX + 1;
  const WaveLds<NMAX> L = wave_carve<NMAX>(smem, R);
  const int l = threadIdx.x;
  const bool act = l < NMAX;
  const size_t ub = blockIdx.x;
  float* Uh = U + ub * cap * DK;
  float* Vh = V + ub * cap * DV;

  for (int w = l; w < NMAX * LDN; w += 64) L.Rb[w] = 0.f;

  // ---- A + B: Gram of U, equilibrated Cholesky --------------------------
  gram_mfma<NMAX, DK>(Uh, n, L.G);
  __syncthreads();
  float g[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) g[i] = act ? L.G[i * LDN + l] : 0.f;
  {
    const float gll = (act && l < n) ? L.G[l * LDN + l] : 0.f;
    const float dl = gll > 0.f ? sqrtf(gll) : 0.f;
    if (act) L.dv[l] = dl;
  }
  __syncthreads();
  {
    const float dl = act ? L.dv[l] : 0.f;
    const float il = dl > 0.f ? 1.f / dl : 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
      const float di = L.dv[i];
      g[i] = di > 0.f ? g[i] * il / di : 0.f;
    }
  }
  // Gram of V into G while the Cholesky runs on registers and Rb
  __syncthreads();
  gram_mfma<NMAX, DV>(Vh, n, L.G);
  for (int j = 0; j < n; ++j) {
    // M[j][l] = M[l][j]: lane j publishes its column, every lane reads its entry
    if (l == j) {
#pragma unroll
      for (int i = 0; i < NMAX; ++i) L.cb[i] = g[i];
    }
    __syncthreads();
    const float gj = act ? L.cb[l] : 0.f;
    const float piv = lane_value(gj, j);
    const bool ok = piv > kPivTol;
    const float p = ok ? sqrtf(piv) : 0.f;
    const float invp = ok ? 1.f / p : 0.f;
    const float r = (l > j && act) ? gj * invp : 0.f;
    if (act) {
      L.Rb[l * LDN + j] = (l == j) ? p : r;   // R[j][l]
      L.wb[l] = r;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NMAX; ++i) g[i] -= L.wb[i] * r;
    __syncthreads();
  }

  // ---- C: H = R G~ R^T with two MFMA products ---------------------------
  //   P = G~ R^T  (into the inverse-iteration region, row stride NMAX)
  //   H = R P     (into G, which G~ no longer needs), then lane l reads
  //   column l of H.
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (act) L.G[i * LDN + l] *= L.dv[i] * L.dv[l];
  __syncthreads();
  {
    constexpr int NT = NMAX / 16;
    const int ci = l & 15, kk = l >> 4;
    float* P = reinterpret_cast<float*>(L.F);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        f4v acc = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NMAX / 4; ++K) {
          const int m = K * 4 + kk;
          const float av = L.G[(I * 16 + ci) * LDN + m];   // G~[i][m]
          const float bv = L.Rb[m * LDN + J * 16 + ci];    // R^T[m][j] = R[j][m]
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) P[(I * 16 + 4 * kk + r) * NMAX + J * 16 + ci] = acc[r];
      }
    __syncthreads();
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        f4v acc = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NMAX / 4; ++K) {
          const int m = K * 4 + kk;
          const float av = L.Rb[m * LDN + I * 16 + ci];    // R[i][m]
          const float bv = P[m * NMAX + J * 16 + ci];      // P[m][j]
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) L.G[(I * 16 + 4 * kk + r) * LDN + J * 16 + ci] = acc[r];
      }
    __syncthreads();
  }
  float h[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) h[i] = act ? L.G[i * LDN + l] : 0.f;
  __syncthreads();

  // ---- D: Householder tridiagonalisation ---------------------------------
  for (int k = 0; k + 2 < n; ++k) {
    // lane k publishes column k; lane i reads H[i][k] (= H[k][i])
    if (l == k) {
#pragma unroll
      for (int i = 0; i < NMAX; ++i) L.cb[i] = h[i];
    }
    __syncthreads();
    const float hk = act ? L.cb[l] : 0.f;
    const float alpha = lane_value(hk, k + 1);
    const float dkk = lane_value(hk, k);
    const float xn2 = wave_sum(l > k + 1 ? hk * hk : 0.f);
    float t, beta, vl;
    if (xn2 == 0.f) {
      t = 0.f;
      beta = alpha;
      vl = (l == k + 1) ? 1.f : 0.f;
    } else {
      beta = -copysignf(sqrtf(alpha * alpha + xn2), alpha);
      t = (beta - alpha) / beta;
      const float sc = 1.f / (alpha - beta);
      vl = (l > k + 1) ? hk * sc : ((l == k + 1) ? 1.f : 0.f);
    }
    if (!act) vl = 0.f;
    if (l == 0) {
      L.td[k] = dkk;
      L.te[k] = beta;
      L.tau[k] = t;
    }
    if (act) {
      L.G[k * LDN + l] = vl;
      L.vb[l] = vl;
    }
    __syncthreads();
    float v[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) v[i] = L.vb[i];
    float pl = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) pl += h[i] * v[i];
    pl *= t;
    const float K = -0.5f * t * wave_sum(pl * vl);
    const float wl = pl + K * vl;
    if (act) L.wb[l] = wl;
    __syncthreads();
    if (l > k) {
#pragma unroll
      for (int i = 0; i < NMAX; ++i) h[i] -= v[i] * wl + L.wb[i] * vl;
    }
    __syncthreads();
  }
  {
    // the trailing 2 x 2 block, from lane n - 1's column
    if (l == n - 1) {
#pragma unroll
      for (int i = 0; i < NMAX; ++i) L.cb[i] = h[i];
    }
    __syncthreads();
    const float e2 = L.cb[n - 2];     // H[n-2][n-1]
    const float d1 = L.cb[n - 1];     // H[n-1][n-1]
    __syncthreads();
    if (l == n - 2) {
#pragma unroll
      for (int i = 0; i < NMAX; ++i) L.cb[i] = h[i];
    }
    __syncthreads();
    const float d2 = L.cb[n - 2];     // H[n-2][n-2]
    if (l == 0) {
      L.td[n - 2] = d2;
      L.te[n - 2] = e2;
      L.td[n - 1] = d1;
      L.te[n - 1] = 0.f;
    }
  }
  __syncthreads();

  // ---- E: the R + 1 largest eigenvalues of T (multisection) -------------
  float tnorm, pivmin;
  {
    float lo_i = 3.0e38f, hi_i = -3.0e38f;
    for (int i = l; i < n; i += 64) {
      const float rad = fabsf(L.te[i]) + (i > 0 ? fabsf(L.te[i - 1]) : 0.f);
      lo_i = fminf(lo_i, L.td[i] - rad);
      hi_i = fmaxf(hi_i, L.td[i] + rad);
    }
    float lo0 = wave_min(lo_i), hi0 = wave_max(hi_i);
    tnorm = fmaxf(fabsf(lo0), fabsf(hi0));
    pivmin = tnorm * 1e-30f + 1e-35f;
    lo0 -= 2.f * kEps * tnorm + pivmin;
    hi0 += 2.f * kEps * tnorm + pivmin;
    const int T = R + 1;
    const int m = 64 / T;                 // lanes per eigenvalue (>= 1)
    const int grp = l / m, sub = l % m;
    const bool live = grp < T;
    const int target = n - 1 - grp;       // ascending index of the eigenvalue
    // pad T to NMAX: diagonal kPadDiag, zero off-diagonal beyond row n - 1
    if (act && l >= n) L.td[l] = kPadDiag;
    if (act && l >= n - 1) L.te[l] = 0.f;
    __syncthreads();
    float dr[NMAX], e2r[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
      dr[i] = L.td[i];
      const float ei = (i > 0) ? L.te[i - 1] : 0.f;
      e2r[i] = ei * ei;
    }
    float lo = lo0, hi = hi0;
    for (int it = 0; it < 64; ++it) {
      const bool done = !live || target < 0 ||
                        (hi - lo) <= 2.f * kEps * fmaxf(fabsf(lo), fabsf(hi)) + pivmin;
      if (__all(done)) break;
      const float pt = lo + (hi - lo) * ((float)(sub + 1) / (float)(m + 1));
      int cnt = 0;
      float q = dr[0] - pt;
      q = (fabsf(q) < pivmin) ? -pivmin : q;
      cnt += (q < 0.f);
#pragma unroll
      for (int i = 1; i < NMAX; ++i) {
        q = (dr[i] - pt) - e2r[i] * __builtin_amdgcn_rcpf(q);
        q = (fabsf(q) < pivmin) ? -pivmin : q;
        cnt += (q < 0.f);
      }
      L.bpt[l] = pt;
      L.bfl[l] = (cnt > target) ? 1 : 0;
      __syncthreads();
      if (live && !done) {
        for (int s = 0; s < m; ++s) {
          const float ps = L.bpt[grp * m + s];
          if (L.bfl[grp * m + s]) hi = fminf(hi, ps);
          else lo = fmaxf(lo, ps);
        }
      }
      __syncthreads();
    }
    if (live && sub == 0) L.lam[grp] = 0.5f * (lo + hi);
  }
  __syncthreads();

  // ---- F: eigenvectors of T by inverse iteration -------------------------
  if (l == 0) {
    // separate equal shifts, then cluster ranks (round in which a vector is computed)
    const float sep = 10.f * kEps * tnorm;
    for (int c = 1; c < R; ++c)
      if (L.lam[c] > L.lam[c - 1] - sep) L.lam[c] = L.lam[c - 1] - sep;
    int maxr = 0;
    for (int c = 0; c < R; ++c) {
      int rk = 0;
      for (int j = 0; j < c; ++j)
        if (fabsf(L.lam[j] - L.lam[c]) < kClusterTol * tnorm && L.rnk[j] + 1 > rk)
          rk = L.rnk[j] + 1;
      L.rnk[c] = rk;
      maxr = rk > maxr ? rk : maxr;
    }
    L.misc[0] = __int_as_float(maxr);
  }
  __syncthreads();
  {
    const int maxr = __float_as_int(L.misc[0]);
    const float tiny = kEps * tnorm + 1e-30f;
    // padded T in registers (td / te were padded in phase E)
    float dr[NMAX], er[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
      dr[i] = L.td[i];
      er[i] = L.te[i];
    }
    const int c = l;
    for (int rnd = 0; rnd <= maxr; ++rnd) {
      if (c < R && L.rnk[c] == rnd) {
        const float lc = L.lam[c];
        float x[NMAX];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c) : 0.f;
        for (int it = 0; it < kInvIters; ++it) {
          // factor T - lc I with partial pivoting while eliminating x; the
          // reciprocal pivot is stored
          float a = dr[0] - lc, b1 = er[0], b2 = 0.f, rr = x[0];
#pragma unroll
          for (int i = 0; i + 1 < NMAX; ++i) {
            const float lw = er[i];
            const float ap = dr[i + 1] - lc;
            const float b1p = (i + 2 < NMAX) ? er[i + 1] : 0.f;
            const float rp = x[i + 1];
            const bool sw = fabsf(lw) > fabsf(a);
            const float pa = sw ? lw : ((a != 0.f) ? a : tiny);
            const float ipa = __builtin_amdgcn_rcpf(pa);
            const float f1 = sw ? ap : b1, f2 = sw ? b1p : b2, fr = sw ? rp : rr;
            L.F[i * R + c] = make_float4(ipa, f1, f2, fr);
            const float mm = sw ? a * ipa : lw * ipa;
            const float na = sw ? (b1 - mm * ap) : (ap - mm * b1);
            const float nb1 = sw ? (b2 - mm * b1p) : (b1p - mm * b2);
            const float nr = sw ? (rr - mm * rp) : (rp - mm * rr);
            a = na; b1 = nb1; b2 = 0.f; rr = nr;
          }
          L.F[(NMAX - 1) * R + c] =
              make_float4(__builtin_amdgcn_rcpf((a != 0.f) ? a : tiny), 0.f, 0.f, rr);
          float x1 = 0.f, x2 = 0.f, mx = 0.f;
#pragma unroll
          for (int i = NMAX - 1; i >= 0; --i) {
            const float4 f = L.F[i * R + c];
            const float xi = (f.w - f.y * x1 - f.z * x2) * f.x;
            x[i] = xi;
            mx = fmaxf(mx, fabsf(xi));
            x2 = x1;
            x1 = xi;
          }
          if (!(mx > 0.f) || !(mx < 3.0e38f)) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c + 7 * it + 1) : 0.f;
            continue;
          }
          const float imx = 1.f / mx;
#pragma unroll
          for (int i = 0; i < NMAX; ++i) x[i] *= imx;
          for (int pass = 0; pass < 2; ++pass) {
            for (int j = 0; j < c; ++j) {
              if (!(fabsf(L.lam[j] - lc) < kClusterTol * tnorm)) continue;
              float dt = 0.f;
#pragma unroll
              for (int i = 0; i < NMAX; ++i)
                if (i < n) dt += x[i] * L.XR[i * R + j];
#pragma unroll
              for (int i = 0; i < NMAX; ++i)
                if (i < n) x[i] -= dt * L.XR[i * R + j];
            }
          }
          float nx = 0.f;
#pragma unroll
          for (int i = 0; i < NMAX; ++i) nx += x[i] * x[i];
          if (nx > 0.f) {
            const float inx = 1.f / sqrtf(nx);
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] *= inx;
          } else {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) x[i] = (i < n) ? start_entry(i, c + 7 * it + 3) : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < NMAX; ++i)
          if (i < n) L.XR[i * R + c] = x[i];
      }
      __syncthreads();
    }
  }

  // one modified Gram-Schmidt pass over the R eigenvectors of T (lane c
  // owns vector c; the current pivot vector is broadcast through cb)
  {
    float x[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) x[i] = (l < R && i < n) ? L.XR[i * R + l] : 0.f;
    for (int c0 = 0; c0 < R; ++c0) {
      if (l == c0) {
#pragma unroll
        for (int i = 0; i < NMAX; ++i) L.cb[i] = x[i];
      }
      __syncthreads();
      float xb[NMAX];
      float nrm2 = 0.f, dt = 0.f;
#pragma unroll
      for (int i = 0; i < NMAX; ++i) {
        xb[i] = L.cb[i];
        nrm2 += xb[i] * xb[i];
        dt += x[i] * xb[i];
      }
      const float inv2 = nrm2 > 0.f ? 1.f / nrm2 : 0.f;
      const float f = (l > c0 && l < R) ? dt * inv2 : 0.f;
      const float sc = (l == c0) ? (nrm2 > 0.f ? 1.f / sqrtf(nrm2) : 0.f) : 1.f;
#pragma unroll
      for (int i = 0; i < NMAX; ++i) x[i] = (x[i] - f * xb[i]) * sc;
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
      if (l < R && i < n) L.XR[i * R + l] = x[i];
  }
  __syncthreads();

  // ---- G + H: X_R = Q Y; P2 = D R^T X_R; T' = D^-1 R^-1 X_R ---------------
  {
    constexpr int CH = NMAX / 2;
    const int c = l & 31, part = l >> 5;
    const bool colok = c < R;
    float y[CH];
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const int i = part * CH + s;
      y[s] = (colok && i < n) ? L.XR[i * R + c] : 0.f;
    }
    for (int k = n - 3; k >= 0; --k) {
      const float tk = L.tau[k];
      float pd = 0.f;
#pragma unroll
      for (int s = 0; s < CH; ++s) pd += L.G[k * LDN + part * CH + s] * y[s];
      const float dt = (pd + __shfl_xor(pd, 32)) * tk;
#pragma unroll
      for (int s = 0; s < CH; ++s) y[s] -= dt * L.G[k * LDN + part * CH + s];
    }
    // P2 = D R^T X_R (R is exactly upper triangular in Rb)
    float* P2 = reinterpret_cast<float*>(L.F);
    for (int j = 0; j < n; ++j) {
      float pd = 0.f;
#pragma unroll
      for (int s = 0; s < CH; ++s) pd += L.Rb[j * LDN + part * CH + s] * y[s];   // R[i][j]
      pd += __shfl_xor(pd, 32);
      if (colok && part == 0) P2[j * R + c] = L.dv[j] * pd;
    }
    // back substitution R t = x, column-oriented; the part owning row i
    // stores t_i / d_i (the row of T') into XR
    for (int i = n - 1; i >= 0; --i) {
      const int own = i / CH, si = i - own * CH;
      float yi = pick(y, si);
      yi = __shfl(yi, c + 32 * own);
      const float rii = L.Rb[i * LDN + i];
      const float ti = rii != 0.f ? yi / rii : 0.f;
      if (colok && part == own) {
        const float di = L.dv[i];
        L.XR[i * R + c] = di > 0.f ? ti / di : 0.f;
      }
#pragma unroll
      for (int s = 0; s < CH; ++s) y[s] -= L.Rb[i * LDN + part * CH + s] * ti;   // R[m][i]
    }
  }
  __syncthreads();

  // ---- I: U' = U T', V' = V P2 as MFMA products --------------------------
  // Tile E covers rows 16 E .. 16 E + 15 of the factor; every read of those
  // rows happens before they are overwritten, and no tile reads another
  // tile's rows, so the products can be written in place.
  {
    const int ci = l & 15, kk = l >> 4;
    constexpr int NK = NMAX / 4;
    constexpr int NC = RMAX / 16;
    const float* P2 = reinterpret_cast<const float*>(L.F);
#pragma unroll
    for (int E = 0; E < DK / 16; ++E) {
      f4v acc[NC];
#pragma unroll
      for (int C = 0; C < NC; ++C) acc[C] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const int j = K * 4 + kk;
        const float av = (j < n) ? Uh[(size_t)j * DK + E * 16 + ci] : 0.f;   // U[e][j]
#pragma unroll
        for (int C = 0; C < NC; ++C) {
          const int cc = C * 16 + ci;
          const float bv = (j < n && cc < R) ? L.XR[j * R + cc] : 0.f;    // T'[j][cc]
          acc[C] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[C], 0, 0, 0);
        }
      }
#pragma unroll
      for (int C = 0; C < NC; ++C) {
        const int cc = C * 16 + ci;
        if (cc < R) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Uh[(size_t)cc * DK + E * 16 + 4 * kk + r] = acc[C][r];
        }
      }
    }
#pragma unroll
    for (int E = 0; E < DV / 16; ++E) {
      f4v acc[NC];
#pragma unroll
      for (int C = 0; C < NC; ++C) acc[C] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const int j = K * 4 + kk;
        const float av = (j < n) ? Vh[(size_t)j * DV + E * 16 + ci] : 0.f;   // V[e][j]
#pragma unroll
        for (int C = 0; C < NC; ++C) {
          const int cc = C * 16 + ci;
          const float bv = (j < n && cc < R) ? P2[j * R + cc] : 0.f;       // P2[j][cc]
          acc[C] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[C], 0, 0, 0);
        }
      }
#pragma unroll
      for (int C = 0; C < NC; ++C) {
        const int cc = C * 16 + ci;
        if (cc < R) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Vh[(size_t)cc * DV + E * 16 + 4 * kk + r] = acc[C][r];
        }
      }
    }
  }
}

template <int NMAX, int DK, int DV, int RMAX>
hipError_t wave_go(int units, int cap, int n, int R, float* U, float* V, hipStream_t s) {
  const size_t bytes = 4 * wave_lds_floats(NMAX, R);
  hipError_t err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(compress_wave_kernel<NMAX, DK, DV, RMAX>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((compress_wave_kernel<NMAX, DK, DV, RMAX>), dim3(units), dim3(64), bytes, s,
                     U, V, cap, n, R);
  return hipGetLastError();
}

template <int DK, int DV, int RMAX>
hipError_t wave_nmax(int units, int cap, int n, int R, float* U, float* V, hipStream_t s) {
  if (n <= 32) return wave_go<32, DK, DV, RMAX>(units, cap, n, R, U, V, s);
  if (n <= 48) return wave_go<48, DK, DV, RMAX>(units, cap, n, R, U, V, s);
  return wave_go<64, DK, DV, RMAX>(units, cap, n, R, U, V, s);
}

template <int DK, int DV>
hipError_t wave_rmax(int units, int cap, int n, int R, float* U, float* V, hipStream_t s) {
  if (R <= 16) return wave_nmax<DK, DV, 16>(units, cap, n, R, U, V, s);
  return wave_nmax<DK, DV, 32>(units, cap, n, R, U, V, s);
}

}  // namespace

size_t compress_wave_lds_bytes(int n, int R) {
  const int nmax = n <= 32 ? 32 : (n <= 48 ? 48 : 64);
  return 4 * wave_lds_floats(nmax, R);
}

hipError_t launch_compress_wave(int batch, int heads, int d_k, int d_v, int cap, int n, int R,
                                float* U, float* V, hipStream_t stream) {
  const int units = batch * heads;
  if (d_k == 128 && d_v == 128) return wave_rmax<128, 128>(units, cap, n, R, U, V, stream);
  if (d_k == 128 && d_v == 64) return wave_rmax<128, 64>(units, cap, n, R, U, V, stream);
  if (d_k == 64 && d_v == 64) return wave_rmax<64, 64>(units, cap, n, R, U, V, stream);
  return hipErrorInvalidValue;
}

}  // namespace seed
