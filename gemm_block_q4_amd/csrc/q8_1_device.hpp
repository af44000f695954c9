// Q8_1 block quantisation arithmetic shared by the quantise kernel and the
// fused gate/up MMQ epilogue, so that both produce the same bytes.
//
// "spark_model/layers/ops/q4k_mmq.rs", quantize_act_q8_1: per 32-value block
// amax = max |x|, d = amax / 127 in binary32, q = rint(x / d) (binary32
// division, round half to even), d stored as binary16 (nearest even) next to
// the exact integer block sum S.  A scale whose binary16 rounding would
// overflow saturates at 65504 and the block is quantised with that stored
// scale.
#pragma once

#include "q4k_device.hpp"

namespace q4k {

// Binary32 scale used for the division (amax is the block's max |x|).
__device__ __forceinline__ float q8_1_scale(float amax) {
  const float d = amax / 127.0f;  // correctly rounded binary32 division
  return d >= 65520.0f ? 65504.0f : d;
}

__device__ __forceinline__ int q8_1_quant(float v, float amax, float d) {
  float r = amax > 0.0f ? rintf(v / d) : 0.0f;
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<int>(r);
}

// Scale/sum word: binary16 d in bits 0-15 (0 for an all-zero block), S in
// bits 16-31.
__device__ __forceinline__ uint32_t q8_1_word(float amax, float d, int s) {
  const uint32_t dbits = amax > 0.0f ? float_to_half_bits(d) : 0u;
  return dbits | (static_cast<uint32_t>(static_cast<uint16_t>(static_cast<int16_t>(s))) << 16);
}

// Four quants as bytes of one word (value 0 in bits 0-7).
__device__ __forceinline__ uint32_t pack_q4(int q0, int q1, int q2, int q3) {
  return (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | ((static_cast<uint32_t>(q3) & 0xFFu) << 24);
}

}  // namespace q4k
