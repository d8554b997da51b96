// Compression kernels for 128 x 64 heads with fp32 factor columns
// (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t compress_wave_128x64(const CompressArgs& args, hipStream_t stream) {
  return wave::wave_dispatch<128, 64, kStoreF32>(args, stream);
}

}  // namespace seed
