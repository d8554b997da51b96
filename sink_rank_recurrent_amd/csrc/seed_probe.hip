// A streaming copy: the bandwidth a plain read-once, write-once kernel gets
// from HBM on this device, measured beside the state kernels so that their
// bandwidth can be set against what the memory system actually delivers
// (as well as against the nominal 8 TB/s).
//
// One 16-byte vector per thread and one workgroup per 4 KiB, plain loads
// and stores.  Of the forms timed on MI355X over 2 GiB (1, 2, 4 or 8
// vectors per thread, grid-stride over 1k to 16k workgroups or a full
// grid, with and without non-temporal hints) this one was fastest, 6.1 TB/s
// read + write.
#include "seed_launch.h"

namespace seed {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 1;   // 16-byte vectors per thread per pass

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const f4* __restrict__ src,
                                                                   f4* __restrict__ dst,
                                                                   size_t n4) {
  const size_t per_block = (size_t)kCopyThreads * kCopyVec;
  const size_t stride = (size_t)gridDim.x * per_block;
  for (size_t base = (size_t)blockIdx.x * per_block + threadIdx.x; base < n4; base += stride) {
    f4 x[kCopyVec];
#pragma unroll
    for (int j = 0; j < kCopyVec; ++j) {
      const size_t e = base + (size_t)j * kCopyThreads;
      if (e < n4) x[j] = src[e];
    }
#pragma unroll
    for (int j = 0; j < kCopyVec; ++j) {
      const size_t e = base + (size_t)j * kCopyThreads;
      if (e < n4) dst[e] = x[j];
    }
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  const size_t per_block = (size_t)kCopyThreads * kCopyVec;
  size_t blocks = (n4 + per_block - 1) / per_block;
  // a full grid; the loop strides only past the largest grid launched
  if (blocks > (size_t)1 << 30) blocks = (size_t)1 << 30;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<const f4*>(src), static_cast<f4*>(dst), n4);
  return hipGetLastError();
}

}  // namespace seed
