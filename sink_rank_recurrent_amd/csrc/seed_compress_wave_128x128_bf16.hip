// Compression kernels for 128 x 128 heads with 16-bit (bf16) kept columns
// (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t compress_wave_128x128_bf16(const CompressArgs& args, hipStream_t stream) {
  return wave::wave_dispatch<128, 128, kStoreBF16>(args, stream);
}

}  // namespace seed
