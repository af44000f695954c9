// Q8_1 activation quantisation for gfx950.
//
// "spark_model/layers/ops/q4k_mmq.rs", quantize_act_q8_1, and "realizar --
// ffn.rs", fused_ffn_swiglu_gpu_true_dp4a (a per-block scale plus 32 int8
// values; quantised once and shared by gate and up).  The per-block
// arithmetic (q8_1_device.hpp): amax = max |x|, d = amax / 127 in binary32,
// q = rint(x / d), d stored as binary16 next to the exact integer block sum.
// The kernel is memory-bound: one lane owns four consecutive values, eight
// lanes (an aligned DPP row quarter) own a block and combine their max and
// sum with three xor shuffles.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"
#include "q8_1_device.hpp"

namespace q4k {

template <bool BF16>
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const void* __restrict__ x,
                                                            int8_t* __restrict__ qs,
                                                            uint32_t* __restrict__ ds,
                                                            size_t groups) {
  const size_t i4 = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  // groups is a multiple of 8 (k % 32 == 0), so an aligned 8-lane group is
  // either wholly inside or wholly outside the range.
  const bool valid = i4 < groups;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    if constexpr (BF16) {
      const uint2 raw = reinterpret_cast<const uint2*>(x)[i4];
      v[0] = bf16_bits_to_float(raw.x & 0xFFFFu);
      v[1] = bf16_bits_to_float(raw.x >> 16);
      v[2] = bf16_bits_to_float(raw.y & 0xFFFFu);
      v[3] = bf16_bits_to_float(raw.y >> 16);
    } else {
      const float4 f = reinterpret_cast<const float4*>(x)[i4];
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
  }
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  const float d = q8_1_scale(amax);
  int q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = q8_1_quant(v[j], amax, d);
  int s = q[0] + q[1] + q[2] + q[3];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  if (valid) {
    reinterpret_cast<uint32_t*>(qs)[i4] = pack_q4(q[0], q[1], q[2], q[3]);
    if ((threadIdx.x & 7) == 0) ds[i4 >> 3] = q8_1_word(amax, d, s);
  }
}

hipError_t launch_q8_1_quantize(const void* x, int x_bf16, int m, int k, int8_t* qs,
                                uint32_t* ds, hipStream_t stream) {
  const size_t groups = static_cast<size_t>(m) * static_cast<size_t>(k) / 4;
  const size_t blocks = (groups + 255) / 256;
  if (x_bf16)
    q8_1_quantize_kernel<true><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(x, qs, ds, groups);
  else
    q8_1_quantize_kernel<false><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(x, qs, ds, groups);
  return hipGetLastError();
}

}  // namespace q4k
