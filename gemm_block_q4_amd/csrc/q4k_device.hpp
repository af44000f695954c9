// Device helpers shared by the gfx950 kernels of the Q4_K FFN library.
//
// block_q4_K (GGML layout, named by "spark_model/layers/ops/q4k_mmq.rs",
// quantize_weight_q4k): bytes 0-1 fp16 d, 2-3 fp16 dmin, 4-15 packed 6-bit
// (scale, min) pairs of the eight 32-weight sub-blocks, 16-143 the quants.
// Read as four 32-bit words, the 16-byte header is
//   h.x = d | dmin << 16, h.y = scales[0..3], h.z = scales[4..7], h.w = scales[8..11].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr int kQK = 256;          // weights per block
constexpr int kBlockBytes = 144;  // bytes per block_q4_K
constexpr int kSub = 32;          // weights per sub-block / values per Q8_1 block
constexpr int kMaxTokens = 8;     // decode regime: tokens per call

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint32_t float_to_half_bits(float v) {
  // v_cvt_f16_f32: round to nearest even, binary16 subnormals kept.
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v)));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// bfloat16 bits of a finite binary32 value, rounded to nearest even
__device__ __forceinline__ uint32_t float_to_bf16_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// 6-bit scale and min of sub-block s (0..7) from the header words.
// Sub-blocks 0-3: scale = low 6 bits of scales[s], min = low 6 bits of
// scales[s+4].  Sub-blocks 4-7: low 4 bits from scales[s+4] (scale: low
// nibble, min: high nibble), high 2 bits from the top of scales[s-4] (scale)
// and scales[s] (min).
template <int S>
__device__ __forceinline__ void scale_min(const uint4& h, uint32_t& sc, uint32_t& mn) {
  static_assert(S >= 0 && S < 8, "sub-block index");
  if constexpr (S < 4) {
    sc = (h.y >> (8 * S)) & 63u;
    mn = (h.z >> (8 * S)) & 63u;
  } else {
    constexpr int U = S - 4;
    sc = ((h.w >> (8 * U)) & 15u) | (((h.y >> (8 * U + 6)) & 3u) << 4);
    mn = ((h.w >> (8 * U + 4)) & 15u) | (((h.z >> (8 * U + 6)) & 3u) << 4);
  }
}

// Runtime sub-block index version (branch-free on the high/low half).
__device__ __forceinline__ void scale_min_rt(const uint4& h, int s, uint32_t& sc, uint32_t& mn) {
  const int u = s & 3;
  const uint32_t b1 = (h.y >> (8 * u)) & 0xFFu;  // scales[u]
  const uint32_t b2 = (h.z >> (8 * u)) & 0xFFu;  // scales[u+4]
  const uint32_t b3 = (h.w >> (8 * u)) & 0xFFu;  // scales[u+8]
  const uint32_t sc_lo = b1 & 63u, mn_lo = b2 & 63u;
  const uint32_t sc_hi = (b3 & 15u) | ((b1 >> 6) << 4);
  const uint32_t mn_hi = (b3 >> 4) | ((b2 >> 6) << 4);
  const bool upper = s >= 4;
  sc = upper ? sc_hi : sc_lo;
  mn = upper ? mn_hi : mn_lo;
}

// Raw buffer loads.  A lane whose byte offset (plus the instruction's
// constant offset) is at or past the resource's size reads zeros and sends no
// memory request, so a load is predicated without a branch.  (A branch around
// a load makes the compiler copy the result at the join, which waits for the
// load right after issuing it and serialises every prefetch.)
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOob = 0x80000000u;  // above every resource size used here
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // 32-bit data format, raw (stride 0) access

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  const v2u32 v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0);
  return make_uint2(v.x, v.y);
}

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u with silu(g) = g / (1 + exp(-g)); for g -> -inf the
  // denominator overflows to +inf and the quotient is -0.
  return g / (1.0f + expf(-g)) * u;
}

}  // namespace q4k
