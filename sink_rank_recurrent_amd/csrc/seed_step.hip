// Fused read-out + exact update of the shallow state (one decode step).
//
// Lemma 2 (SEED summary on picx.dev, "Exact Update (Lemma 2)"), with the
// Kimi Delta Attention form taking Diag(g) for the scalar decay and the
// Mamba-2 form being Lemma 1 with Phi = g I:
//   omega = v.vbar/|vbar|^2,  eps = v - omega vbar
//   a+ = G a + beta (omega - k.(G a)) k          (Mamba-2: g a + omega k)
//   U+ = [G U, k]
//   V+ = [V, beta (eps - V (G U)^T k)]            (Mamba-2: [V, eps])
//   o  = vbar (a+.q) + V+ (U+^T q)               (read-out after the update)
//
// Mapping on gfx950: one 512-thread workgroup (8 wave64s) per (request,
// head).  The workgroup is NG = 16 column groups of 32 lanes (half-waves).
// Group c owns factor columns j = c, c+16, c+32, ...; inside a column each
// lane holds d_k/32 consecutive entries of the U column and d_v/32 of the V
// column, so every load and store is a coalesced 8- or 16-byte access per
// lane.  All U and V columns are loaded into registers at the start (the
// state is read exactly once), so the only dependent step is the reduction
// of c_k = (G U)^T k and c_q = (G U)^T q inside each half-wave, which then
// feeds that half-wave's own V columns without any exchange.  The 16
// partial V-sums are combined through LDS.  Every half-wave recomputes the
// scalars (omega, k.Ga, k.q, a+.q) from its own copy of the small vectors,
// which avoids a barrier; only group 0 writes a, the new V column and o.
// With 16 groups a thread holds at most ceil(r/16) <= 3 columns below 48
// held columns (<= 64 VGPRs), so 8 waves fit a SIMD: 1024 units run at once
// and a launch of 8192 units is exactly 8 rounds.  The factor columns are
// loaded and stored non-temporally: in a model every other layer's state
// streams through before this one is touched again.
//
// LAZY: the decay of U is kept as a running product gam per unit (per key
// channel for Kimi Delta Attention) instead of being applied in place: the
// stored columns are U~ with U = Diag(gam) U~.  A step multiplies gam by g,
// reads U~ without rewriting it (c_k = U~^T (gam k), c_q = U~^T (gam q))
// and appends U~_r = k / gam.  The arithmetic is Lemma 2's; only the U
// write-back disappears.
//
// The running product must stay a normal fp32 number (k / gam is appended).
// When a channel's product after this step falls below kFoldBelow = 2^-64,
// the step applies it to that row of every held column -- the in-place
// decay, for that channel -- and restarts the product at 1.  In the
// per-request schedule's interval between a snapshot and its merge the
// held columns may still be read by the snapshot's compression, so there
// is no fold; a product below kPoisonBelow = 2^-110 in that interval makes
// the unit's decay product NaN, which every later read-out carries.
//
// FMT != kStoreF32 (16-bit kept factors, always with LAZY): columns j < kR
// are the 16-bit patterns the last compression rounded (SEED figures and
// tables, Table 4 and Table 9: factors rounded at every compression) and are
// widened exactly on load; columns j >= kR, appended since, are fp32 at
// index j - kR of U and V.  A step writes a 16-bit column only to fold a
// vanishing decay product into it (rounded to nearest).
#include "seed_device.h"
#include "seed_launch.h"

namespace seed {

constexpr float kFoldBelow = 0x1p-64f;
constexpr float kPoisonBelow = 0x1p-110f;
// Lazily decayed launches (fp32, 16-bit or ring layout) of at least this
// many units and at most 80 held columns use 8 column groups (256 threads)
// per workgroup: 4 to 8 units share a CU instead of 3 or 4.  The form decayed in
// place keeps 16 groups (its U write-back fills the combine phase), as do
// small batches, which 16 groups spread over more of the GPU.
constexpr int kHalfGroupUnits = 2048;

template <int RULE, int DK, int DV, typename IN_T, int NG, int SLOTS, bool LAZY, int FMT>
__global__ __launch_bounds__(32 * NG) void seed_step_kernel(
    float* __restrict__ a, float* __restrict__ U, float* __restrict__ V,
    uint16_t* __restrict__ Uk, const uint16_t* __restrict__ Vk, float* __restrict__ gam,
    const float* __restrict__ vbar, const IN_T* __restrict__ q, const IN_T* __restrict__ k,
    const IN_T* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ o, int heads, int cap, int r_arg, int kR_arg, RingArgs rg) {
  static_assert(FMT == kStoreF32 || LAZY, "16-bit kept columns are never decayed in place");
  constexpr bool RING = FMT == kStoreRing;
  constexpr bool H16 = FMT == kStoreBF16 || FMT == kStoreF16;
  constexpr int EK = DK / 32;  // key-space entries per lane
  constexpr int EV = DV / 32;  // value-space entries per lane
  const int kR = H16 ? kR_arg : 0;
  const int unit = blockIdx.x;
  const int h = unit % heads;
  const int tid = threadIdx.x;
  const int grp = tid >> 5;
  const int lane = tid & 31;
  const size_t ub = (size_t)unit;
  // fp32 columns j >= kR at index j - kR (the ring: see column())
  float* Uh = U + ub * cap * DK;
  float* Vh = V + ub * cap * DV;

  // the ring layout's per-request schedule (RingArgs in seed_launch.h)
  int r = r_arg;
  int win0 = 0;
  bool merge = false, snap = false, pending = false;
  float* keptU = nullptr;
  float* keptV = nullptr;
  if constexpr (RING) {
    const int A = rg.t - rg.t_start[unit / heads];
    if (A < 0) {
      // not started: the state is left as it is, the read-out is zero
      if (tid < DV) o[ub * DV + tid] = 0.f;
      return;
    }
    const int c = (A < rg.W + rg.D) ? 0 : (A - rg.D) / rg.W;
    win0 = c * rg.W;
    r = kR_arg + A - win0;
    merge = c >= 1 && A == win0 + rg.D;
    snap = (A + 1) % rg.W == 0;
    // a snapshot taken and not yet merged: its compression may read the
    // held columns
    pending = A >= rg.W && A % rg.W < rg.D;
    const size_t kb = ((size_t)(c & 1) * gridDim.x + ub) * kR_arg;
    keptU = rg.KU + kb * DK;
    keptV = rg.KV + kb * DV;
  }
  // fp32 column j of U / V
  auto ucol = [&](int j) -> float* {
    if constexpr (RING)
      return j < kR_arg ? keptU + (size_t)j * DK : Uh + (size_t)((win0 + j - kR_arg) % cap) * DK;
    else
      return Uh + (size_t)(j - kR) * DK;
  };
  auto vcol = [&](int j) -> float* {
    if constexpr (RING)
      return j < kR_arg ? keptV + (size_t)j * DV : Vh + (size_t)((win0 + j - kR_arg) % cap) * DV;
    else
      return Vh + (size_t)(j - kR) * DV;
  };

  // 1. the factors: every column this half-wave owns, loaded once
  float u[SLOTS][EK];
  float w[SLOTS][EV];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int j = grp + NG * s;
    if (H16 && j < r && j < kR) {
      load_vec16_nt<FMT, EK>(Uk + (ub * kR + j) * DK + lane * EK, u[s]);
      load_vec16_nt<FMT, EV>(Vk + (ub * kR + j) * DV + lane * EV, w[s]);
    } else if (j < r) {
      load_vec_nt<EK>(ucol(j) + lane * EK, u[s]);
      load_vec_nt<EV>(vcol(j) + lane * EV, w[s]);
    } else {
#pragma unroll
      for (int e = 0; e < EK; ++e) u[s][e] = 0.f;
#pragma unroll
      for (int e = 0; e < EV; ++e) w[s][e] = 0.f;
    }
  }

  // 2. the step's inputs and the sink coefficient
  float kk[EK], qq[EK], aa[EK], gk[EK];
  load_vec<EK>(k + ub * DK + lane * EK, kk);
  load_vec<EK>(q + ub * DK + lane * EK, qq);
  load_vec<EK>(a + ub * DK + lane * EK, aa);
  float gs = 1.f;
  if constexpr (RULE == kKDA) {
    load_vec<EK>(g + ub * DK + lane * EK, gk);
  } else {
    gs = g[ub];
#pragma unroll
    for (int e = 0; e < EK; ++e) gk[e] = gs;
  }
  // LAZY: the running decay product after this step, and k, q scaled by it
  float gn[EK];
  float kx[EK], qx[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    gn[e] = 1.f;
    kx[e] = kk[e];
    qx[e] = qq[e];
  }
  if constexpr (LAZY) {
    if constexpr (RULE == kKDA) {
      load_vec<EK>(gam + ub * DK + lane * EK, gn);
    } else {
      const float g0 = gam[ub];
#pragma unroll
      for (int e = 0; e < EK; ++e) gn[e] = g0;
    }
    // gm: the product that scales this step's sums over the loaded columns
    // (the old product times g).  Folds -- at a merge, or of a vanishing
    // product -- rewrite the stored columns only: the loaded ones are never
    // modified, so neither their old values nor their addresses stay live
    // beside the new ones (19 fewer VGPRs in the ring layout at 7 slots).
    // gp: the scale the stored columns now carry against the loaded ones.
    float gm[EK], gp[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      gm[e] = gn[e] * gk[e];
      gp[e] = 1.f;
    }
    if constexpr (RING) {
      if (merge) {
        // fold the decay product into every held column, then restart it
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
          const int j = grp + NG * s;
          if (j < r) {
            float x[EK];
#pragma unroll
            for (int e = 0; e < EK; ++e) x[e] = u[s][e] * gn[e];
            store_vec<EK>(ucol(j) + lane * EK, x);
          }
        }
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          gp[e] = gn[e];
          gn[e] = 1.f;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) gn[e] *= gk[e];
    // a vanishing product: fold it into this row of every held column
    bool fold[EK];
    bool any = false;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      fold[e] = gn[e] < kFoldBelow;
      any = any || fold[e];
    }
    if (pending) {
#pragma unroll
      for (int e = 0; e < EK; ++e)
        if (gn[e] < kPoisonBelow) gn[e] = gm[e] = __builtin_nanf("");
    } else if (any) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int j = grp + NG * s;
        if (j < r) {
          // the folded rows carry the whole product, gm (= gp gn)
          float x[EK];
#pragma unroll
          for (int e = 0; e < EK; ++e) x[e] = u[s][e] * (fold[e] ? gm[e] : gp[e]);
          if (H16 && j < kR)
            store_vec16_nearest<FMT, EK>(Uk + (ub * kR + j) * DK + lane * EK, x);
          else
            store_vec<EK>(ucol(j) + lane * EK, x);
        }
      }
#pragma unroll
      for (int e = 0; e < EK; ++e)
        if (fold[e]) gn[e] = 1.f;
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      kx[e] = gm[e] * kk[e];
      qx[e] = gm[e] * qq[e];
    }
  }
  float bt = 1.f;
  if constexpr (RULE != kMAMBA2) bt = beta[ub];
  float vv[EV], vb[EV];
  load_vec<EV>(v + ub * DV + lane * EV, vv);
  load_vec<EV>(vbar + (size_t)h * DV + lane * EV, vb);

  // 3. value split: omega = v.vbar / |vbar|^2
  float p_vvb = 0.f, p_nvb = 0.f;
#pragma unroll
  for (int e = 0; e < EV; ++e) {
    p_vvb += vv[e] * vb[e];
    p_nvb += vb[e] * vb[e];
  }
  const float omega = sum32(p_vvb) / sum32(p_nvb);

  // 4. sink coefficient
  float ga[EK];
  float p_kga = 0.f, p_kq = 0.f;
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    ga[e] = gk[e] * aa[e];
    p_kga += kk[e] * ga[e];
    p_kq += kk[e] * qq[e];
  }
  const float kq = sum32(p_kq);
  float an[EK];
  if constexpr (RULE == kMAMBA2) {
#pragma unroll
    for (int e = 0; e < EK; ++e) an[e] = ga[e] + omega * kk[e];
  } else {
    const float coef = bt * (omega - sum32(p_kga));
#pragma unroll
    for (int e = 0; e < EK; ++e) an[e] = ga[e] + coef * kk[e];
  }
  float p_aq = 0.f;
#pragma unroll
  for (int e = 0; e < EK; ++e) p_aq += an[e] * qq[e];
  const float aq = sum32(p_aq);

  // 5. U pass: decay in place (each decayed column is stored as soon as it
  // is formed, and the appended column U_r = k with them), then
  // c_k = (G U)^T k and c_q = (G U)^T q
  float ck[SLOTS], cq[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    float pk = 0.f, pq = 0.f;
    if constexpr (LAZY) {
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        pk += u[s][e] * kx[e];
        pq += u[s][e] * qx[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const float x = gk[e] * u[s][e];
        u[s][e] = x;
        pk += x * kk[e];
        pq += x * qq[e];
      }
      const int j = grp + NG * s;
      if (j < r) store_vec_nt<EK>(ucol(j) + lane * EK, u[s]);
    }
    ck[s] = pk;
    cq[s] = pq;
  }
  if (grp == r % NG) {
    if constexpr (LAZY) {
      float kd[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) kd[e] = kk[e] / gn[e];
      store_vec_nt<EK>(ucol(r) + lane * EK, kd);
    } else {
      store_vec_nt<EK>(ucol(r) + lane * EK, kk);
    }
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    if constexpr (RULE != kMAMBA2) ck[s] = sum32(ck[s]);
    cq[s] = sum32(cq[s]);
  }

  // 6. V pass: partial V c_k and V c_q over this half-wave's columns
  float sk[EV], sq[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) {
    sk[e] = 0.f;
    sq[e] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      if constexpr (RULE != kMAMBA2) sk[e] += w[s][e] * ck[s];
      sq[e] += w[s][e] * cq[s];
    }
  }

  // 7. combine the column groups through LDS: thread e < d_v finishes
  // value entry e (a short tail: 2 kGroups partial sums per thread)
  __shared__ float red[2][NG][DV];
  __shared__ float eps_s[DV], sink_s[DV];
#pragma unroll
  for (int e = 0; e < EV; ++e) {
    red[0][grp][lane * EV + e] = sk[e];
    red[1][grp][lane * EV + e] = sq[e];
  }
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      eps_s[lane * EV + e] = vv[e] - omega * vb[e];
      sink_s[lane * EV + e] = vb[e] * aq;
    }
    store_vec<EK>(a + ub * DK + lane * EK, an);
    if constexpr (LAZY) {
      if constexpr (RULE == kKDA) store_vec<EK>(gam + ub * DK + lane * EK, gn);
      else if (lane == 0) gam[ub] = gn[0];
    }
    if constexpr (RING) {
      if (snap) {
        if constexpr (RULE == kKDA) store_vec<EK>(rg.gam_snap + ub * DK + lane * EK, gn);
        else if (lane == 0) rg.gam_snap[ub] = gn[0];
      }
    }
  }
  __syncthreads();
  if (tid < DV) {
    float tk = 0.f, tq = 0.f;
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      tk += red[0][c][tid];
      tq += red[1][c][tid];
    }
    const float eps = eps_s[tid];
    const float vn = (RULE == kMAMBA2) ? eps : bt * (eps - tk);
    __builtin_nontemporal_store(vn, vcol(r) + tid);
    o[ub * DV + tid] = sink_s[tid] + tq + vn * kq;
  }
}

namespace {

struct StepArgs {
  RingArgs ring;
  int units, heads, cap, r, kR;
  float* a;
  float* U;
  float* V;
  uint16_t* Uk;
  const uint16_t* Vk;
  float* gam;
  const float* vbar;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* o;
};

template <int RULE, int DK, int DV, typename IN_T, int NG, int SLOTS, bool LAZY, int FMT>
void step_launch(const StepArgs& p, hipStream_t s) {
  hipLaunchKernelGGL((seed_step_kernel<RULE, DK, DV, IN_T, NG, SLOTS, LAZY, FMT>), dim3(p.units),
                     dim3(32 * NG), 0, s, p.a, p.U, p.V, p.Uk, p.Vk, p.gam, p.vbar,
                     static_cast<const IN_T*>(p.q), static_cast<const IN_T*>(p.k),
                     static_cast<const IN_T*>(p.v), p.g, p.beta, p.o, p.heads, p.cap, p.r, p.kR,
                     p.ring);
}

template <int RULE, int DK, int DV, typename IN_T, int NG, int SLOTS>
hipError_t step_go(int fmt, const StepArgs& p, hipStream_t s) {
  if (fmt == kStoreRing) {
    step_launch<RULE, DK, DV, IN_T, NG, SLOTS, true, kStoreRing>(p, s);
  } else if (fmt == kStoreBF16) {
    step_launch<RULE, DK, DV, IN_T, NG, SLOTS, true, kStoreBF16>(p, s);
  } else if (fmt == kStoreF16) {
    step_launch<RULE, DK, DV, IN_T, NG, SLOTS, true, kStoreF16>(p, s);
  } else if (p.gam != nullptr) {
    step_launch<RULE, DK, DV, IN_T, NG, SLOTS, true, kStoreF32>(p, s);
  } else {
    step_launch<RULE, DK, DV, IN_T, NG, SLOTS, false, kStoreF32>(p, s);
  }
  return hipGetLastError();
}

template <int RULE, int DK, int DV, typename IN_T>
hipError_t step_slots(int fmt, const StepArgs& p, hipStream_t s) {
  static_assert(6 * 16 >= kMaxCap, "slot instances cover the capacity");
  if (p.gam != nullptr && p.units >= kHalfGroupUnits && p.r <= 10 * 8) {
    const int need = (p.r + 7) / 8;
#define SEED_STEP_SLOTS(N) \
    if (need <= N) return step_go<RULE, DK, DV, IN_T, 8, N>(fmt, p, s);
    SEED_STEP_SLOTS(1)
    SEED_STEP_SLOTS(2)
    SEED_STEP_SLOTS(3)
    SEED_STEP_SLOTS(4)
    SEED_STEP_SLOTS(5)
    SEED_STEP_SLOTS(6)
    SEED_STEP_SLOTS(7)
    SEED_STEP_SLOTS(8)
    SEED_STEP_SLOTS(9)
    SEED_STEP_SLOTS(10)
#undef SEED_STEP_SLOTS
  }
  const int need = (p.r + 15) / 16;
#define SEED_STEP_SLOTS(N) \
  if (need <= N) return step_go<RULE, DK, DV, IN_T, 16, N>(fmt, p, s);
  SEED_STEP_SLOTS(1)
  SEED_STEP_SLOTS(2)
  SEED_STEP_SLOTS(3)
  SEED_STEP_SLOTS(4)
  SEED_STEP_SLOTS(5)
  SEED_STEP_SLOTS(6)
#undef SEED_STEP_SLOTS
  return hipErrorInvalidValue;
}

template <int RULE, typename IN_T>
hipError_t step_dims(int d_k, int d_v, int fmt, const StepArgs& p, hipStream_t s) {
  if (d_k == 128 && d_v == 128) return step_slots<RULE, 128, 128, IN_T>(fmt, p, s);
  if (d_k == 128 && d_v == 64) return step_slots<RULE, 128, 64, IN_T>(fmt, p, s);
  if (d_k == 64 && d_v == 64) return step_slots<RULE, 64, 64, IN_T>(fmt, p, s);
  return hipErrorInvalidValue;
}

template <int RULE>
hipError_t step_dtype(bool bf16, int d_k, int d_v, int fmt, const StepArgs& p, hipStream_t s) {
  if (bf16) return step_dims<RULE, bf16_t>(d_k, d_v, fmt, p, s);
  return step_dims<RULE, float>(d_k, d_v, fmt, p, s);
}

}  // namespace

hipError_t launch_step(int rule, bool in_bf16, int store_fmt, int batch, int heads, int d_k,
                       int d_v, int cap, int r, int kR, float* a, float* U, float* V,
                       uint16_t* Uk, const uint16_t* Vk, float* gam, const float* vbar,
                       const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float* o, hipStream_t stream, const RingArgs* ring) {
  if (store_fmt != kStoreF32 && gam == nullptr) return hipErrorInvalidValue;
  if (store_fmt == kStoreRing && ring == nullptr) return hipErrorInvalidValue;
  const RingArgs rg = ring != nullptr ? *ring : RingArgs{nullptr, 0, 1, 0, nullptr, nullptr, nullptr};
  const StepArgs p{rg, batch * heads, heads, cap, r, store_fmt == kStoreF32 ? 0 : kR, a, U, V, Uk,
                   Vk, gam, vbar, q, k, v, g, beta, o};
  switch (rule) {
    case kGDN: return step_dtype<kGDN>(in_bf16, d_k, d_v, store_fmt, p, stream);
    case kKDA: return step_dtype<kKDA>(in_bf16, d_k, d_v, store_fmt, p, stream);
    case kMAMBA2: return step_dtype<kMAMBA2>(in_bf16, d_k, d_v, store_fmt, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace seed
