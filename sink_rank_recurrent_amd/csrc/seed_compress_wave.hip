// Host dispatch of the wave compression kernel (seed_compress_wave.h) by
// head shape and storage format; each (shape, format) pair is compiled in
// its own source file.
#include "seed_compress_wave.h"
#include "seed_launch.h"

namespace seed {

size_t compress_wave_lds_bytes(int n, int R) { return wave::wave_lds_bytes_for(n, R); }

size_t compress_lds_bytes(int n, int R) { return compress_wave_lds_bytes(n, R); }

hipError_t launch_compress(int d_k, int d_v, int store_fmt, const CompressArgs& args,
                           hipStream_t stream) {
#define SEED_COMPRESS_SHAPE(DK, DV)                                              \
  if (d_k == DK && d_v == DV) {                                                  \
    if (store_fmt == kStoreF32) return compress_wave_##DK##x##DV(args, stream);  \
    if (store_fmt == kStoreBF16) return compress_wave_##DK##x##DV##_bf16(args, stream); \
    if (store_fmt == kStoreF16) return compress_wave_##DK##x##DV##_fp16(args, stream);  \
    if (store_fmt == kStoreRing) return compress_wave_##DK##x##DV##_ring(args, stream);  \
    return hipErrorInvalidValue;                                                 \
  }
  SEED_COMPRESS_SHAPE(128, 128)
  SEED_COMPRESS_SHAPE(128, 64)
  SEED_COMPRESS_SHAPE(64, 64)
#undef SEED_COMPRESS_SHAPE
  return hipErrorInvalidValue;
}

size_t convert_lds_bytes(int d_k, int R) { return wave::convert_lds_bytes_for(d_k, R); }

hipError_t launch_convert(int d_k, int d_v, const CompressArgs& args, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return convert_wave_128x128(args, stream);
  if (d_k == 128 && d_v == 64) return convert_wave_128x64(args, stream);
  if (d_k == 64 && d_v == 64) return convert_wave_64x64(args, stream);
  return hipErrorInvalidValue;
}

}  // namespace seed
