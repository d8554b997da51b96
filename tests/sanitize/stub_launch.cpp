// Host-only stand-ins for the device launchers of seed_launch.h, so that
// the C ABI's host validation (seed_api.cpp) can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a
// GPU.  Test infrastructure: every launcher enqueues nothing and reports
// success; the LDS queries accept every shape; the statistics record has
// the library's 16 fields.
#include "seed_launch.h"

namespace seed {

hipError_t launch_step(int, bool, int, int, int, int, int, int, int, int, float*, float*, float*,
                       uint16_t*, const uint16_t*, float*, const float*, const void*, const void*,
                       const void*, const float*, const float*, float*, hipStream_t,
                       const RingArgs*) {
  return hipSuccess;
}
hipError_t launch_dense(int, bool, int, int, int, int, float*, const void*, const void*,
                        const void*, const float*, const float*, float*, hipStream_t) {
  return hipSuccess;
}
size_t compress_lds_bytes(int, int) { return 0; }
size_t compress_wave_lds_bytes(int, int) { return 0; }
size_t stats_lds_bytes(int, int) { return 0; }
size_t convert_lds_bytes(int, int) { return 0; }
hipError_t launch_convert(int, int, const CompressArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_compress(int, int, int, const CompressArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_round_factors(int, int, int, int, int, const float*, const float*, uint16_t*,
                                uint16_t*, int, uint32_t, uint32_t, uint32_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_handoff(bool, int, int, int, int, int, int, int, int, const int*, float*, void*,
                          void*, void*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_join(int, int, int, int, int, int, int, int, int, const int*, const void*, float*,
                       float*, float*, float*, hipStream_t) {
  return hipSuccess;
}
int stat_fields() { return 16; }
hipError_t launch_state_stats(int, int, int, int, int, const float*, const float*, float*, float*,
                              float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_stream_copy(const void*, void*, size_t, hipStream_t) { return hipSuccess; }

}  // namespace seed
