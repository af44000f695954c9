// Q8_1 activation quantisation for gfx950.
//
// "spark_model/layers/ops/q4k_mmq.rs", quantize_act_q8_1, and "realizar --
// ffn.rs", fused_ffn_swiglu_gpu_true_dp4a (a per-block scale plus 32 int8
// values; quantised once and shared by gate and up).  The per-block
// arithmetic (q8_1_device.hpp): amax = max |x|, d = amax / 127 in binary32,
// q = rint(x / d), d stored as binary16 next to the exact integer block sum.
// One lane owns four consecutive values; eight lanes (half a DPP row) own a
// block and combine their max and sum with three register-level lane
// exchanges.  The codes q = rint(x / d) come from a reciprocal multiply when
// that provably gives the same integer: with v_rcp_f32 (1 ulp) the product p
// is within 1.6 * 2^-23 |t| of t = x / d and binary32 t within 2^-24 |t|,
// i.e. less than 2^-15 apart where |t| <= 127.5 matters, so p more than 2^-14
// from every half-integer rounds like the correctly rounded quotient.  A
// wavefront with a near-tie, or with a scale below the binary32 normal range
// (whose reciprocal overflows), takes the division.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"
#include "q8_1_device.hpp"

namespace q4k {

namespace {

// v of lane ^ 1, ^ 2 and ^ 4 (DPP; lanes outside BANKS keep old)
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, 0xF,
                                                           BANKS, false));
}
__device__ __forceinline__ uint32_t xor1_u(uint32_t v) { return dpp_u<0xB1, 0xF>(v, v); }  // quad_perm(1,0,3,2)
__device__ __forceinline__ uint32_t xor2_u(uint32_t v) { return dpp_u<0x4E, 0xF>(v, v); }  // quad_perm(2,3,0,1)
__device__ __forceinline__ uint32_t xor4_u(uint32_t v) {
  return dpp_u<0x114, 0xA>(dpp_u<0x104, 0x5>(v, v), v);  // row_shl:4 into banks 0, 2; row_shr:4 into 1, 3
}
__device__ __forceinline__ float xor1_f(float v) { return __uint_as_float(xor1_u(__float_as_uint(v))); }
__device__ __forceinline__ float xor2_f(float v) { return __uint_as_float(xor2_u(__float_as_uint(v))); }
__device__ __forceinline__ float xor4_f(float v) { return __uint_as_float(xor4_u(__float_as_uint(v))); }

}  // namespace

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
  amax = fmaxf(amax, xor1_f(amax));
  amax = fmaxf(amax, xor2_f(amax));
  amax = fmaxf(amax, xor4_f(amax));
  const float d = q8_1_scale(amax);
  int q[4];
  {
    const bool fast = d >= 0x1p-126f;  // an all-zero block has d = 0 and codes 0
    const float inv = fast ? __builtin_amdgcn_rcpf(d) : 0.0f;
    bool slow = amax > 0.0f && !fast;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = v[j] * inv;
      const float r = rintf(p);
      slow |= fabsf(fabsf(p - r) - 0.5f) <= 0x1p-14f;
      q[j] = static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f));
    }
    if (__any(slow)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = q8_1_quant(v[j], amax, d);
    }
  }
  int s = q[0] + q[1] + q[2] + q[3];
  s += static_cast<int>(xor1_u(static_cast<uint32_t>(s)));
  s += static_cast<int>(xor2_u(static_cast<uint32_t>(s)));
  s += static_cast<int>(xor4_u(static_cast<uint32_t>(s)));
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
