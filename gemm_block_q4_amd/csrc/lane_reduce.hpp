// Cross-lane sums on the VALU for the GEMV kernels (gfx950): DPP moves and
// the lane swaps between half-waves (v_permlane32_swap) and between rows of
// 16 lanes (v_permlane16_swap).  No LDS round trip; fixed summation order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

// Lane permute (DPP).  Lanes whose source is out of range read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, true));
}

// Sum over the 64 lanes, landing in lane 63: within quads, then rows of 16
// (row_shr 4, 8), then across rows (row_bcast 15 and 31).
__device__ __forceinline__ float wave_total_last(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm(1,0,3,2)
  v += dpp_f<0x4E>(v);        // quad_perm(2,3,0,1)
  v += dpp_f<0x114>(v);       // row_shr:4
  v += dpp_f<0x118>(v);       // row_shr:8
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Lane swaps across the two half-waves (permlane32) and across the rows of
// each half-wave (permlane16): the pair (a, b) comes back as two registers
// whose sum, in every lane, adds one operand over the two swapped lane sets,
// a in one half (or row pair) and b in the other.  Summing pairs this way
// halves the number of values per reduction step.
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sums over the 64 lanes of MT values per lane with the value count halved
// per step (two swap levels, then DPP within rows of 16).  Lanes flagged by
// token_map hold a total; fixed order, deterministic.
template <int MT>
__device__ __forceinline__ float row_reduce(const float (&acc)[MT], int lane) {
  if constexpr (MT == 1) {
    return wave_total_last(acc[0]);
  } else {
    float w[MT / 2];
#pragma unroll
    for (int j = 0; j < MT / 2; ++j) w[j] = swap_sum32(acc[2 * j], acc[2 * j + 1]);
    float y;
    if constexpr (MT == 2) {
      y = w[0];
    } else {
      float x[MT / 4];
#pragma unroll
      for (int i = 0; i < MT / 4; ++i) x[i] = swap_sum16(w[2 * i], w[2 * i + 1]);
      if constexpr (MT == 4) {
        y = x[0];
      } else {
        // lanes 8..15 of each row keep x1, lanes 0..7 keep x0 (row_ror:8 is
        // the lane xor 8 within a row)
        const bool b3 = (lane >> 3) & 1;
        const float send = b3 ? x[0] : x[1], keep = b3 ? x[1] : x[0];
        y = keep + dpp_f<0x128>(send);
      }
    }
    if constexpr (MT != 8) y += dpp_f<0x128>(y);  // row_ror:8
    y += dpp_f<0xB1>(y);                           // quad_perm(1,0,3,2)
    y += dpp_f<0x4E>(y);                           // quad_perm(2,3,0,1)
    y += dpp_f<0x114>(y);                          // row_shr:4: lanes 4..7 of each half-row
    if constexpr (MT == 2) y += dpp_f<0x142, 0xA>(y);  // row_bcast:15 into rows 1, 3
    return y;
  }
}

// Which value's total row_reduce leaves in this lane, found once by running
// the same swaps on value indices; holder marks one lane per value.
template <int MT>
__device__ __forceinline__ void token_map(int lane, int& tok, bool& holder) {
  if constexpr (MT == 1) {
    tok = 0;
    holder = lane == 63;
  } else {
    uint32_t w[MT / 2];
#pragma unroll
    for (int j = 0; j < MT / 2; ++j) w[j] = __builtin_amdgcn_permlane32_swap(2u * j, 2u * j + 1u, false, false)[0];
    if constexpr (MT == 2) {
      tok = static_cast<int>(w[0]);
      holder = (lane & 31) == 31;
    } else {
      uint32_t x[MT / 4];
#pragma unroll
      for (int i = 0; i < MT / 4; ++i) x[i] = __builtin_amdgcn_permlane16_swap(w[2 * i], w[2 * i + 1], false, false)[0];
      if constexpr (MT == 4) {
        tok = static_cast<int>(x[0]);
        holder = (lane & 15) == 15;
      } else {
        tok = static_cast<int>((lane >> 3) & 1 ? x[1] : x[0]);
        holder = (lane & 7) == 7;
      }
    }
  }
}

}  // namespace q4k
