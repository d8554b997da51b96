// Host-side launchers of the gfx950 kernels.  They assume validated
// arguments (seed_api.cpp checks everything first) and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace seed {

// Largest factor capacity (R + W) the kernels are compiled for.
constexpr int kMaxCap = 96;
// LDS available to one workgroup on gfx950.
constexpr size_t kMaxLds = 160 * 1024;

// gam == NULL: U decayed in place; otherwise the lazily decayed form
// U = Diag(gam) U~ (gam per key channel for KDA, one scalar per unit else).
hipError_t launch_step(int rule, bool in_bf16, int batch, int heads, int d_k, int d_v, int cap,
                       int r, float* a, float* U, float* V, float* gam, const float* vbar, const void* q,
                       const void* k, const void* v, const float* g, const float* beta, float* o,
                       hipStream_t stream);

hipError_t launch_dense(int rule, bool in_bf16, int batch, int heads, int d_k, int d_v, float* S,
                        const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float* o, hipStream_t stream);

// Largest column count the wave compression kernel handles (one wave per
// unit up to 64 columns, two above).
constexpr int kWaveMaxN = 96;

// Dynamic LDS bytes the compression of n columns to rank R needs.
size_t compress_lds_bytes(int n, int R);
size_t compress_wave_lds_bytes(int n, int R);
// Dynamic LDS bytes the dense-to-shallow kernel needs.
size_t from_dense_lds_bytes(int d_k, int R);

// Compression of n <= kWaveMaxN columns to rank R (seed_compress_wave.h).
// gam as for launch_step (NULL: U at true scale); it is reset to 1.
hipError_t launch_compress(int batch, int heads, int d_k, int d_v, int cap, int n, int R,
                           float* U, float* V, float* gam, int gam_per_row, hipStream_t stream);
hipError_t launch_compress_wave(int batch, int heads, int d_k, int d_v, int cap, int n, int R,
                                float* U, float* V, float* gam, int gam_per_row,
                                hipStream_t stream);
hipError_t compress_wave_128x128(int units, int cap, int n, int R, float* U, float* V, float* gam,
                                 int gam_per_row, hipStream_t stream);
hipError_t compress_wave_128x64(int units, int cap, int n, int R, float* U, float* V, float* gam,
                                int gam_per_row, hipStream_t stream);
hipError_t compress_wave_64x64(int units, int cap, int n, int R, float* U, float* V, float* gam,
                               int gam_per_row, hipStream_t stream);

hipError_t launch_from_dense(int batch, int heads, int d_k, int d_v, int cap, int R,
                             const float* S, const float* vbar, float* a, float* U, float* V,
                             hipStream_t stream);

}  // namespace seed
