// End-of-prefill conversion of 128 x 128 dense states by the compression
// kernel's eigensolver (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t convert_wave_128x128(const CompressArgs& args, hipStream_t stream) {
  return wave::convert_dispatch<128, 128>(args, stream);
}

}  // namespace seed
