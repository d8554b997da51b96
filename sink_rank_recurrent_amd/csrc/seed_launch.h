// Host-side launchers of the gfx950 kernels.  They assume validated
// arguments (seed_api.cpp checks everything first) and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace seed {

// Storage of the factor columns: all fp32, or the R columns the last
// compression wrote as 16-bit patterns (bf16 or fp16) and the rest fp32.
// kStoreRing: per-request schedules -- R kept fp32 columns in one of two
// buffers, the window in a ring of W + D columns (seed_sched.hip's layout).
// kConvert is not a storage format but the compression kernel's other use:
// the end-of-prefill conversion of dense states (launch_convert).
enum StoreFmt { kStoreF32 = 0, kStoreBF16 = 1, kStoreF16 = 2, kStoreRing = 3, kConvert = 4 };

// Per-request schedule of the ring layout.  A request b has taken
// A = t - t_start[b] steps (it is idle while A < 0).  With
// c = A < W + D ? 0 : (A - D) / W merges done, its kept columns are buffer
// c & 1 of KU / KV ([2][units][R][d]); window column i (0 <= i < A - c W) is
// column number c W + i, stored in ring slot (c W + i) mod (W + D); the step
// appends column number A.  The step with A = c W + D (c >= 1) first folds
// the running decay product into every held column and resets it to 1; the
// step with (A + 1) mod W == 0 also writes the decay product to gam_snap.
struct RingArgs {
  const int* t_start;
  int t, W, D;
  float* KU;
  float* KV;
  float* gam_snap;
};

// Largest factor capacity (R + W) the kernels are compiled for.
constexpr int kMaxCap = 96;
// LDS available to one workgroup on gfx950.
constexpr size_t kMaxLds = 160 * 1024;

// gam == NULL: U decayed in place; otherwise the lazily decayed form
// U = Diag(gam) U~ (gam per key channel for KDA, one scalar per unit else).
// store_fmt (StoreFmt) kStoreF32: every column in U, V (capacity cap);
// kStoreBF16 / kStoreF16: columns j < kR are the 16-bit Uk, Vk ([unit][kR]
// columns) and columns j >= kR are U, V at index j - kR (capacity cap);
// these need gam.
// kStoreRing: U, V are the rings (cap = W + D columns), kR = R, r the
// largest column count any request holds (R + W + D - 1), ring describes the
// schedule.
hipError_t launch_step(int rule, bool in_bf16, int store_fmt, int batch, int heads, int d_k,
                       int d_v, int cap, int r, int kR, float* a, float* U, float* V,
                       uint16_t* Uk, const uint16_t* Vk, float* gam, const float* vbar,
                       const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float* o, hipStream_t stream,
                       const RingArgs* ring = nullptr);

hipError_t launch_dense(int rule, bool in_bf16, int batch, int heads, int d_k, int d_v, float* S,
                        const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float* o, hipStream_t stream);

// Largest column count the wave compression kernel handles (one wave per
// unit up to 64 columns, two above).
constexpr int kWaveMaxN = 96;

// Dynamic LDS bytes the compression of n columns to rank R needs.
size_t compress_lds_bytes(int n, int R);
size_t compress_wave_lds_bytes(int n, int R);
// Dynamic LDS bytes the statistics kernel needs.
size_t stats_lds_bytes(int d_k, int R);

// Arguments of the compression of n <= kWaveMaxN columns to rank R
// (seed_compress_wave.h).  fp32 layout (Uk == NULL): columns 0..n-1 in U, V
// (capacity cap), the result written in place to columns 0..R-1.  16-bit
// layout: columns 0..R-1 are the patterns in Uk, Vk ([unit][R] columns) and
// columns R..n-1 are U, V at index j - R (capacity cap); the result is
// rounded into Uk, Vk (to nearest, or stochastically with the Philox words
// of (unit, epoch, key)).  gam as for launch_step (NULL: U at true scale);
// it is reset to 1.
// Ring layout (kStoreRing, per-request schedules): block i compresses unit
// list[i]; a unit whose request has A = t_snap - t_start[b] steps with
// k = A / W >= 1 and A - k W < max(D, 1) (its snapshot k taken, not yet
// merged) compresses its kept buffer (k - 1) & 1 and window column numbers
// (k - 1) W .. k W - 1 (ring U, V with cap = W + D slots), with gam the
// decay product at the snapshot, into kept buffer k & 1 scaled by 1 / gam;
// gam is not reset.  Other units of the list are left alone.
struct CompressArgs {
  int units, cap, n, R;
  float* U;
  float* V;
  uint16_t* Uk;
  uint16_t* Vk;
  float* gam;
  int gam_per_row;
  int stochastic;
  uint32_t epoch, key_lo, key_hi;
  const int* list;
  const int* t_start;
  int heads, t_snap, W, D, units_total;
  float* KU;
  float* KV;
  // conversion (kConvert): dense states S [units][d_k][d_v], vbar [heads][d_v];
  // writes a [units][d_k] and columns 0..R-1 of U, V (capacity cap)
  const float* S;
  const float* vbar;
  float* a;
};

// End-of-prefill conversion by the compression kernel's eigensolver:
// H = C C^T = S S^T - |vbar|^2 a a^T (n = d_k columns), U' = its top-R
// eigenvectors, V' = C^T U' = S^T U' - vbar (a^T U').
hipError_t launch_convert(int d_k, int d_v, const CompressArgs& args, hipStream_t stream);
size_t convert_lds_bytes(int d_k, int R);
#define SEED_DECLARE_CONVERT_SHAPE(DK, DV) \
  hipError_t convert_wave_##DK##x##DV(const CompressArgs& args, hipStream_t stream);
SEED_DECLARE_CONVERT_SHAPE(128, 128)
SEED_DECLARE_CONVERT_SHAPE(128, 64)
SEED_DECLARE_CONVERT_SHAPE(64, 64)
#undef SEED_DECLARE_CONVERT_SHAPE

hipError_t launch_compress(int d_k, int d_v, int store_fmt, const CompressArgs& args,
                           hipStream_t stream);
#define SEED_DECLARE_COMPRESS_SHAPE(DK, DV)                                                    \
  hipError_t compress_wave_##DK##x##DV(const CompressArgs& args, hipStream_t stream);          \
  hipError_t compress_wave_##DK##x##DV##_bf16(const CompressArgs& args, hipStream_t stream);   \
  hipError_t compress_wave_##DK##x##DV##_fp16(const CompressArgs& args, hipStream_t stream);   \
  hipError_t compress_wave_##DK##x##DV##_ring(const CompressArgs& args, hipStream_t stream);
SEED_DECLARE_COMPRESS_SHAPE(128, 128)
SEED_DECLARE_COMPRESS_SHAPE(128, 64)
SEED_DECLARE_COMPRESS_SHAPE(64, 64)
#undef SEED_DECLARE_COMPRESS_SHAPE

// Rounds fp32 rank-R factors U [unit][R][d_k], V [unit][R][d_v] into the
// 16-bit Uk, Vk (same layouts), element numbering and words as in the
// compression.
hipError_t launch_round_factors(int store_fmt, int units, int R, int d_k, int d_v, const float* U,
                                const float* V, uint16_t* Uk, uint16_t* Vk, int stochastic,
                                uint32_t epoch, uint32_t key_lo, uint32_t key_hi,
                                hipStream_t stream);

// Copies the rank-R states of the units of requests idx[0..n_sel) between
// the state arrays (a fp32; U, V with cap columns of factor_bytes entries)
// and the packed buffer (seed_handoff.hip); pack: state -> buffer.
hipError_t launch_handoff(bool pack, int batch, int heads, int d_k, int d_v, int cap, int R,
                          int factor_bytes, int n_sel, const int* idx, float* a, void* U, void* V,
                          void* buf, hipStream_t stream);

// Unpack of fp32 rank-R states into batch slots slot[0..n_sel) of a batch
// that holds r >= R columns: a and columns 0..R-1 from buf, columns R..r-1
// zeroed, and gam (gam_len floats per unit, 0: none) set to 1.
hipError_t launch_join(int batch, int heads, int d_k, int d_v, int cap, int R, int r, int gam_len,
                       int n_sel, const int* slot, const void* buf, float* a, float* U, float* V,
                       float* gam, hipStream_t stream);

// Statistics of dense states (seed_stats.hip): stat_fields() floats per
// unit in rec; the sorted eigenvalues of S S^T and C C^T in specS, specC
// ([unit][d_k], either may be NULL).
int stat_fields();
hipError_t launch_state_stats(int batch, int heads, int d_k, int d_v, int R, const float* S,
                              const float* vbar, float* rec, float* specS, float* specC,
                              hipStream_t stream);

// Streaming copy of `bytes` (a multiple of 16, 16-byte aligned buffers that
// do not overlap), the bandwidth probe of seed_probe.hip.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace seed
