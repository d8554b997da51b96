// End-of-prefill conversion of 64 x 64 dense states by the compression
// kernel's eigensolver (kernel template in seed_compress_wave.h).
#include "seed_compress_wave.h"

namespace seed {

hipError_t convert_wave_64x64(const CompressArgs& args, hipStream_t stream) {
  return wave::convert_dispatch<64, 64>(args, stream);
}

}  // namespace seed
