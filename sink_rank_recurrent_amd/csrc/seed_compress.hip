// Statistics of dense states by cyclic Jacobi (seed_state_stats).
//
// A dense state S splits into its sink a = S vbar/|vbar|^2 (SEED figures and
// tables on thelatestinai.com, Fig. 3 (b)) and content C = S - a vbar^T.
// The statistics need whole spectra of S S^T and C C^T and their top
// eigenvectors to full accuracy, once per inspected state, so one 256-thread
// workgroup per unit diagonalises each d_k x d_k Gram in LDS by cyclic
// Jacobi with parallel ordering, run to convergence.  (The end-of-prefill
// conversion, which needs only the top R, runs on the compression kernel's
// tridiagonal eigensolver in seed_compress_wave.h.)
#include "seed_device.h"
#include "seed_launch.h"

namespace seed {

namespace {

constexpr int kNT = 256;
constexpr int kChunk = 32;          // rows staged per Gram pass
constexpr float kRotTol = 1e-6f;    // rotate when |h_pq| > kRotTol sqrt(h_pp h_qq)
constexpr int kMaxSweeps = 15;

struct Lds {
  int np, ld;     // padded order (even) and row stride
  float* H;       // [np][ld]  G_V, then the core H (Jacobi works here)
  float* X;       // [max(np,kChunk)][ld]  Gram staging, then P, then eigenvectors
  float* T;       // [np][R]   X_R, then R^{-1} X_R scaled
  float* cs;      // [np]      (c, s) per pair
  int* pq;        // [np]      (p, q) per pair
  int* rank;      // [np]      descending rank of H_ii
  float* aux;     // [256]     sink coefficient and vbar (dense conversion)
  int* flag;      // [4]
};

__host__ __device__ inline int padded(int n) { return n + (n & 1); }

__host__ __device__ inline size_t lds_floats(int np, int R) {
  const int ld = np + 1;
  const int xrows = np > kChunk ? np : kChunk;
  size_t f = 0;
  f += (size_t)np * ld;                   // H
  f += (size_t)xrows * ld;                // X
  f += (size_t)np * R;                    // T
  f += 2 * (size_t)np;                    // cs, pq
  f += np;                                // rank
  f += 256 + 4;                           // aux, flag
  return f;
}

__device__ inline Lds carve(float* base, int n, int R) {
  Lds L;
  L.np = padded(n);
  L.ld = L.np + 1;
  const int xrows = L.np > kChunk ? L.np : kChunk;
  float* p = base;
  L.H = p; p += (size_t)L.np * L.ld;
  L.X = p; p += (size_t)xrows * L.ld;
  L.T = p; p += (size_t)L.np * R;
  L.cs = p; p += L.np;
  L.pq = reinterpret_cast<int*>(p); p += L.np;
  L.rank = reinterpret_cast<int*>(p); p += L.np;
  L.aux = p; p += 256;
  L.flag = reinterpret_cast<int*>(p);
  return L;
}

// out[i][j] = sum_e col_i[e] col_j[e] for i, j < n, where col(j, e) yields
// entry e of column j (0 <= e < d).  Register-blocked: thread (ti, tj) of a
// 16 x 16 grid owns a BS x BS block.  Columns are staged kChunk entries at a
// time in `stage` as [entry][column].
template <int BS, typename ColFn>
__device__ __forceinline__ void gram(ColFn col, int n, int d, float* out, int ld, float* stage) {
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tj = tid & 15;
  float acc[BS][BS];
#pragma unroll
  for (int x = 0; x < BS; ++x)
#pragma unroll
    for (int y = 0; y < BS; ++y) acc[x][y] = 0.f;
  for (int e0 = 0; e0 < d; e0 += kChunk) {
    for (int idx = tid; idx < kChunk * n; idx += kNT) {
      const int j = idx / kChunk, e = idx % kChunk;
      stage[e * ld + j] = (e0 + e < d) ? col(j, e0 + e) : 0.f;
    }
    __syncthreads();
    for (int e = 0; e < kChunk; ++e) {
      float xi[BS], xj[BS];
#pragma unroll
      for (int x = 0; x < BS; ++x) {
        const int i = ti * BS + x, j = tj * BS + x;
        xi[x] = i < n ? stage[e * ld + i] : 0.f;
        xj[x] = j < n ? stage[e * ld + j] : 0.f;
      }
#pragma unroll
      for (int x = 0; x < BS; ++x)
#pragma unroll
        for (int y = 0; y < BS; ++y) acc[x][y] += xi[x] * xj[y];
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < BS; ++x)
#pragma unroll
    for (int y = 0; y < BS; ++y) {
      const int i = ti * BS + x, j = tj * BS + y;
      if (i < n && j < n) out[i * ld + j] = acc[x][y];
    }
}

template <typename ColFn>
__device__ __forceinline__ void gram_dispatch(ColFn col, int n, int d, float* out, int ld, float* stage) {
  const int bs = (n + 15) / 16;
  if (bs <= 2) gram<2>(col, n, d, out, ld, stage);
  else if (bs <= 3) gram<3>(col, n, d, out, ld, stage);
  else if (bs <= 4) gram<4>(col, n, d, out, ld, stage);
  else if (bs <= 6) gram<6>(col, n, d, out, ld, stage);
  else gram<8>(col, n, d, out, ld, stage);
}

__device__ inline void rr_pair(int t, int i, int np, int& p, int& q) {
  const int m = np - 1;
  int x, y;
  if (i == 0) {
    x = m;
    y = t;
  } else {
    x = (t + i) % m;
    y = (t - i + m) % m;
  }
  p = x < y ? x : y;
  q = x < y ? y : x;
}

// Ranks of the diagonal of H (descending; ties by index) into L.rank.
__device__ __forceinline__ void rank_diagonal(const Lds& L) {
  const int tid = threadIdx.x;
  for (int i = tid; i < L.np; i += kNT) {
    const float di = L.H[i * L.ld + i];
    int r = 0;
    for (int j = 0; j < L.np; ++j) {
      const float dj = L.H[j * L.ld + j];
      r += (dj > di) || (dj == di && j < i);
    }
    L.rank[i] = r;
  }
}

// Cyclic Jacobi on the symmetric L.H (np x np, padding zero), accumulating
// eigenvectors into L.X (set to the identity here).  On exit the diagonal
// of H holds the eigenvalues and L.rank their descending ranks.  Stops when
// every off-diagonal entry is at most full_tol.
__device__ __forceinline__ void jacobi(const Lds& L, float full_tol) {
  const int tid = threadIdx.x;
  const int np = L.np, ld = L.ld, nb = np / 2;
  float* H = L.H;
  float* X = L.X;
  for (int w = tid; w < np * np; w += kNT) {
    const int i = w / np, j = w % np;
    X[i * ld + j] = (i == j) ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    for (int t = 0; t < np - 1; ++t) {
      for (int i = tid; i < nb; i += kNT) {
        int p, q;
        rr_pair(t, i, np, p, q);
        const float app = H[p * ld + p], aqq = H[q * ld + q], apq = H[p * ld + q];
        float c = 1.f, s = 0.f;
        if (apq != 0.f && fabsf(apq) > kRotTol * sqrtf(fabsf(app * aqq))) {
          const float tau = (aqq - app) / (2.f * apq);
          const float tt = copysignf(1.f, tau) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + tt * tt);
          s = tt * c;
        }
        L.cs[2 * i] = c;
        L.cs[2 * i + 1] = s;
        L.pq[2 * i] = p;
        L.pq[2 * i + 1] = q;
      }
      __syncthreads();
      // H <- J^T H J, one 2x2 block (I, J) at a time with I <= J; the
      // mirrored block is written from the same values, so H stays exactly
      // symmetric.
      for (int w = tid; w < nb * nb; w += kNT) {
        const int I = w / nb, J = w % nb;
        if (I > J) continue;
        const int p1 = L.pq[2 * I], q1 = L.pq[2 * I + 1];
        const int p2 = L.pq[2 * J], q2 = L.pq[2 * J + 1];
        const float c1 = L.cs[2 * I], s1 = L.cs[2 * I + 1];
        const float c2 = L.cs[2 * J], s2 = L.cs[2 * J + 1];
        if (s1 == 0.f && s2 == 0.f) continue;
        const float b00 = H[p1 * ld + p2], b01 = H[p1 * ld + q2];
        const float b10 = H[q1 * ld + p2], b11 = H[q1 * ld + q2];
        const float x00 = c1 * b00 - s1 * b10, x01 = c1 * b01 - s1 * b11;
        const float x10 = s1 * b00 + c1 * b10, x11 = s1 * b01 + c1 * b11;
        float y00 = c2 * x00 - s2 * x01, y01 = s2 * x00 + c2 * x01;
        float y10 = c2 * x10 - s2 * x11, y11 = s2 * x10 + c2 * x11;
        if (I == J) {
          y01 = 0.f;
          y10 = 0.f;
        }
        H[p1 * ld + p2] = y00;
        H[p1 * ld + q2] = y01;
        H[q1 * ld + p2] = y10;
        H[q1 * ld + q2] = y11;
        if (I != J) {
          H[p2 * ld + p1] = y00;
          H[q2 * ld + p1] = y01;
          H[p2 * ld + q1] = y10;
          H[q2 * ld + q1] = y11;
        }
      }
      for (int w = tid; w < np * nb; w += kNT) {
        const int e = w / nb, I = w % nb;
        const float s = L.cs[2 * I + 1];
        if (s == 0.f) continue;
        const float c = L.cs[2 * I];
        const int p = L.pq[2 * I], q = L.pq[2 * I + 1];
        const float xp = X[e * ld + p], xq = X[e * ld + q];
        X[e * ld + p] = c * xp - s * xq;
        X[e * ld + q] = s * xp + c * xq;
      }
      __syncthreads();
    }
    rank_diagonal(L);
    if (tid == 0) L.flag[0] = 0;
    __syncthreads();
    bool bad = false;
    for (int w = tid; w < np * np; w += kNT) {
      const int i = w / np, j = w % np;
      if (i != j && fabsf(H[i * ld + j]) > full_tol) bad = true;
    }
    if (bad) L.flag[0] = 1;
    __syncthreads();
    if (L.flag[0] == 0) break;
    __syncthreads();
  }
}

// Statistics of dense states (SEED figures and tables: Fig. 3 (e), (g),
// (h); Fig. 12 (f); Fig. 13 (a), (b), (d)).  Per unit: the sink split
// a = S vbar / |vbar|^2; the energies |S|^2 (trace of S S^T), |a vbar^T|^2 =
// |a|^2 |vbar|^2 and |C|^2; the eigenvectors x_i of S S^T and of C C^T by
// Jacobi run to convergence, each eigenvalue then taken as the Rayleigh
// quotient |M^T x_i|^2 from the matrix itself (second order in the
// eigenvector's error, so fp32 Jacobi's drift on the diagonal does not
// enter); v* = S^T x_1 / |S^T x_1|; the smallest ranks holding 90 % and 99 %
// of the content's energy and the share beyond rank R.  Record per unit
// (kStatFields floats): e_state, e_sink, e_content, sink share, top share,
// |cos(v*, vbar)|, rank90, rank99, share beyond R, then zeros.
constexpr int kStatFields = 16;
constexpr float kFullTol = 1e-7f;   // off-diagonal / trace at convergence

// M (DK x DV, row j from mrow(j, e)) into the rows of L.H, after a Jacobi
// has finished with it.
template <int DK, int DV, typename RowFn>
__device__ __forceinline__ void stage_rows(const Lds& L, RowFn mrow) {
  __syncthreads();
  for (int w = threadIdx.x; w < DK * DV; w += kNT) {
    const int j = w / DV, e = w % DV;
    L.H[j * L.ld + e] = mrow(j, e);
  }
  __syncthreads();
}

// lam[i] = |M^T x_i|^2 for the columns x_i of L.X (M staged in L.H); two
// groups of threads split the value entries, their partial sums meet in
// p0 and p1 (DK floats each).  Then rank[i] = descending rank of lam[i].
template <int DK, int DV>
__device__ __forceinline__ void rayleigh(const Lds& L, float* p0, float* p1, float* lam,
                                         int* rank) {
  const int tid = threadIdx.x;
  const int i = tid % DK, half = tid / DK;
  if (half < 2) {
    float acc = 0.f;
    for (int e = half * (DV / 2); e < (half + 1) * (DV / 2); ++e) {
      float y = 0.f;
      for (int j = 0; j < DK; ++j) y += L.H[j * L.ld + e] * L.X[j * L.ld + i];
      acc += y * y;
    }
    (half ? p1 : p0)[i] = acc;
  }
  __syncthreads();
  for (int k = tid; k < DK; k += kNT) lam[k] = p0[k] + p1[k];
  __syncthreads();
  for (int k = tid; k < DK; k += kNT) {
    int r = 0;
    for (int j = 0; j < DK; ++j) r += (lam[j] > lam[k]) || (lam[j] == lam[k] && j < k);
    rank[k] = r;
  }
  __syncthreads();
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void stats_kernel(const float* __restrict__ S,
                                                     const float* __restrict__ vbar, int heads,
                                                     int R, float* __restrict__ rec,
                                                     float* __restrict__ specS,
                                                     float* __restrict__ specC) {
  extern __shared__ float smem[];
  const Lds L = carve(smem, DK, 1);
  const int tid = threadIdx.x;
  const int ld = L.ld;
  const size_t ub = blockIdx.x;
  const int h = (int)(ub % heads);
  const float* Sh = S + ub * DK * DV;
  float* av = L.aux;          // [DK] sink coefficient
  float* vb = L.aux + 128;    // [DV] vbar
  // after a Jacobi: cs and pq hold the two partial sums, T the eigenvalues
  // (np * 1 floats), rank their order
  float* p0 = L.cs;
  float* p1 = reinterpret_cast<float*>(L.pq);
  float* lam = L.T;

  for (int e = tid; e < DV; e += kNT) vb[e] = vbar[(size_t)h * DV + e];
  __syncthreads();
  float nv2 = 0.f;
  for (int e = 0; e < DV; ++e) nv2 += vb[e] * vb[e];
  {
    constexpr int EV = DV / 32;
    const int grp = tid >> 5, lane = tid & 31;
    for (int i = grp; i < DK; i += 8) {
      float x[EV];
      load_vec<EV>(Sh + (size_t)i * DV + lane * EV, x);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EV; ++e) p += x[e] * vb[lane * EV + e];
      p = sum32(p) / nv2;
      if (lane == 0) av[i] = p;
    }
  }
  __syncthreads();
  float na = 0.f;
  for (int i = 0; i < DK; ++i) na += av[i] * av[i];
  const float e_sink = na * nv2;
  float* out = rec + ub * kStatFields;

  // S S^T: spectrum of S and its top direction
  gram_dispatch([=](int j, int e) { return Sh[(size_t)j * DV + e]; }, DK, DV, L.H, ld, L.X);
  __syncthreads();
  // the trace, summed by every thread in the same order
  float e_state = 0.f;
  for (int i = 0; i < DK; ++i) e_state += L.H[i * ld + i];
  jacobi(L, kFullTol * e_state);
  stage_rows<DK, DV>(L, [=](int j, int e) { return Sh[(size_t)j * DV + e]; });
  rayleigh<DK, DV>(L, p0, p1, lam, L.rank);
  int i0 = 0;
  for (int i = 0; i < DK; ++i)
    if (L.rank[i] == 0) i0 = i;
  if (specS != nullptr)
    for (int i = tid; i < DK; i += kNT) specS[ub * DK + L.rank[i]] = lam[i];
  // v* = S^T x_1 (value space): its direction against vbar
  for (int e = tid; e < DV; e += kNT) {
    float y = 0.f;
    for (int j = 0; j < DK; ++j) y += L.H[j * ld + e] * L.X[j * ld + i0];
    p0[e] = y;
  }
  __syncthreads();
  if (tid == 0) {
    float nn = 0.f, dot = 0.f;
    for (int e = 0; e < DV; ++e) {
      nn += p0[e] * p0[e];
      dot += p0[e] * vb[e];
    }
    out[0] = e_state;
    out[1] = e_sink;
    out[3] = e_state > 0.f ? e_sink / e_state : 0.f;
    out[4] = e_state > 0.f ? lam[i0] / e_state : 0.f;
    out[5] = (nn > 0.f && nv2 > 0.f) ? fabsf(dot) / sqrtf(nn * nv2) : 0.f;
    for (int f = 9; f < kStatFields; ++f) out[f] = 0.f;
  }
  __syncthreads();

  // C C^T: spectrum of the content
  gram_dispatch([=](int j, int e) { return Sh[(size_t)j * DV + e] - av[j] * vb[e]; }, DK, DV, L.H,
                ld, L.X);
  __syncthreads();
  float e_content = 0.f;
  for (int i = 0; i < DK; ++i) e_content += L.H[i * ld + i];
  jacobi(L, kFullTol * e_content);
  stage_rows<DK, DV>(L, [=](int j, int e) { return Sh[(size_t)j * DV + e] - av[j] * vb[e]; });
  rayleigh<DK, DV>(L, p0, p1, lam, L.rank);
  for (int i = tid; i < DK; i += kNT) {
    p0[L.rank[i]] = lam[i];
    if (specC != nullptr) specC[ub * DK + L.rank[i]] = lam[i];
  }
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int i = 0; i < DK; ++i) tot += p0[i];
    int r90 = 0, r99 = 0;
    float c = 0.f, beyond = 0.f;
    for (int i = 0; i < DK; ++i) {
      c += p0[i];
      if (r90 == 0 && tot > 0.f && c >= 0.90f * tot) r90 = i + 1;
      if (r99 == 0 && tot > 0.f && c >= 0.99f * tot) r99 = i + 1;
      if (i >= R) beyond += p0[i];
    }
    out[2] = e_content;
    out[6] = (float)r90;
    out[7] = (float)r99;
    out[8] = tot > 0.f ? beyond / tot : 0.f;
  }
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int DK, int DV>
hipError_t stats_go(int units, int heads, int R, const float* S, const float* vbar, float* rec,
                    float* specS, float* specC, hipStream_t s) {
  const size_t bytes = stats_lds_bytes(DK, 1);
  hipError_t err = set_lds(stats_kernel<DK, DV>, bytes);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((stats_kernel<DK, DV>), dim3(units), dim3(kNT), bytes, s, S, vbar, heads, R,
                     rec, specS, specC);
  return hipGetLastError();
}

}  // namespace

size_t compress_lds_bytes(int n, int R) { return compress_wave_lds_bytes(n, R); }

int stat_fields() { return kStatFields; }

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

size_t stats_lds_bytes(int d_k, int R) { return 4 * lds_floats(padded(d_k), R); }

}  // namespace seed
