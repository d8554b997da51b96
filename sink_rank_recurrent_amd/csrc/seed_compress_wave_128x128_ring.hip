// Compression kernels for 128 x 128 heads in the ring layout of per-request
// schedules (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t compress_wave_128x128_ring(const CompressArgs& args, hipStream_t stream) {
  return wave::wave_dispatch<128, 128, kStoreRing>(args, stream);
}

}  // namespace seed
