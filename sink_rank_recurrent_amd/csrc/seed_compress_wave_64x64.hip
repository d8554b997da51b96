// Compression kernels for 64 x 64 heads (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t compress_wave_64x64(int units, int cap, int n, int R, float* U, float* V, float* gam,
                              int gam_per_row, hipStream_t stream) {
  return wave::wave_dispatch<64, 64>(units, cap, n, R, U, V, gam, gam_per_row, stream);
}

}  // namespace seed
