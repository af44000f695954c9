// Q8_1 activation quantisation for gfx950.
//
// "spark_model/layers/ops/q4k_mmq.rs", quantize_act_q8_1, and "realizar --
// ffn.rs", fused_ffn_swiglu_gpu_true_dp4a (a per-block scale plus 32 int8
// values; quantised once and shared by gate and up).  Per 32-value block:
// amax = max |x|, d = amax / 127 in binary32, q = rint(x / d) (binary32
// division, round half to even), stored d as binary16 (nearest even) and the
// exact integer block sum S (a scale that would overflow binary16 saturates
// at 65504 and quantises the block).  The kernel is memory-bound: one lane owns four
// consecutive values, eight lanes (an aligned DPP row quarter) own a block and
// combine their max and sum with three xor shuffles.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

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
  float d = amax / 127.0f;  // correctly rounded binary32 division
  // A scale whose binary16 rounding would overflow saturates at the largest
  // finite binary16 value, and the block is quantised with that stored scale.
  if (d >= 65520.0f) d = 65504.0f;
  int q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r = amax > 0.0f ? rintf(v[j] / d) : 0.0f;
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    q[j] = static_cast<int>(r);
  }
  int s = q[0] + q[1] + q[2] + q[3];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  if (valid) {
    const uint32_t packed = (static_cast<uint32_t>(q[0]) & 0xFFu) |
                            ((static_cast<uint32_t>(q[1]) & 0xFFu) << 8) |
                            ((static_cast<uint32_t>(q[2]) & 0xFFu) << 16) |
                            ((static_cast<uint32_t>(q[3]) & 0xFFu) << 24);
    reinterpret_cast<uint32_t*>(qs)[i4] = packed;
    if ((threadIdx.x & 7) == 0) {
      const uint32_t dbits = amax > 0.0f ? float_to_half_bits(d) : 0u;
      ds[i4 >> 3] = dbits | (static_cast<uint32_t>(static_cast<uint16_t>(static_cast<int16_t>(s))) << 16);
    }
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
