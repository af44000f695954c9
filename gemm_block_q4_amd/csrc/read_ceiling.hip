// Plain-read ceiling: the time a trivial kernel needs to stream a buffer from
// HBM, measured beside the GEMV on the same rotated weight copies so that the
// GEMV's share of what the device can stream per launch is known.  One
// 16-byte load per thread, 256 threads per workgroup (the fastest of the
// plain read shapes measured on gfx950: more loads per thread, larger
// workgroups and grid-stride loops were all slower per launch); the loaded
// words feed a comparison so the loads cannot be dropped, and the sink is
// written only if the XOR of a lane's 16 bytes equals a fixed value.
#include <hip/hip_runtime.h>

#include "q4k_internal.hpp"

namespace q4k {

namespace {

__global__ __launch_bounds__(256) void read_ceiling_kernel(const uint4* __restrict__ p, size_t n16,
                                                           uint32_t* __restrict__ sink) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 v = p[i];
  if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9E3779B9u) sink[0] = static_cast<uint32_t>(i);
}

}  // namespace

hipError_t launch_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = (n16 + 255) / 256;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  read_ceiling_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace q4k
