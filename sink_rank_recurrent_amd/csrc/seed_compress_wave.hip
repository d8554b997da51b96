// Host dispatch of the wave compression kernel (seed_compress_wave.h) by
// head shape; each shape is compiled in its own source file.
#include "seed_compress_wave.h"
#include "seed_launch.h"

namespace seed {

size_t compress_wave_lds_bytes(int n, int R) { return wave::wave_lds_bytes_for(n, R); }

hipError_t launch_compress_wave(int batch, int heads, int d_k, int d_v, int cap, int n, int R,
                                float* U, float* V, float* gam, int gam_per_row,
                                hipStream_t stream) {
  const int units = batch * heads;
  if (d_k == 128 && d_v == 128)
    return compress_wave_128x128(units, cap, n, R, U, V, gam, gam_per_row, stream);
  if (d_k == 128 && d_v == 64)
    return compress_wave_128x64(units, cap, n, R, U, V, gam, gam_per_row, stream);
  if (d_k == 64 && d_v == 64)
    return compress_wave_64x64(units, cap, n, R, U, V, gam, gam_per_row, stream);
  return hipErrorInvalidValue;
}

}  // namespace seed
