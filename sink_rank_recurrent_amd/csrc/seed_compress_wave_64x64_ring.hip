// Compression kernels for 64 x 64 heads in the ring layout of per-request
// schedules (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t compress_wave_64x64_ring(const CompressArgs& args, hipStream_t stream) {
  return wave::wave_dispatch<64, 64, kStoreRing>(args, stream);
}

}  // namespace seed
