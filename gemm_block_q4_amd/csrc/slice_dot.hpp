// Device helpers of the activation-stationary Q4_K GEMV (one activation row
// held per lane as integer digits), shared by the dense / MoE-pair kernel and
// the expert-major MoE kernels, gfx950.
//
// A row of a Q4_K matrix is cut into 4*(k/256) slices of 64 weights (quarter
// g of a 256-block: quant bytes 32g..32g+31, low nibbles = sub-block 2g, high
// nibbles = sub-block 2g+1).  A lane owns one slice position and holds that
// slice of the activations as integer digits: a power-of-two scale 2^e with
// every |x| < 2^e and a = rint(x * 2^(21-e)) (21 significant bits relative to
// the slice maximum), stored as two unsigned byte planes and one signed plane
// (a = u0 + 2^8 u1 + 2^16 (u2 - 64)).  Four weights times one plane are one
// v_dot4; the plane sums of a sub-block combine exactly in int32, scaled by
// 2^(e-21), and the min term uses the f32 sums of the slice's two halves.
#pragma once

#include "lane_reduce.hpp"
#include "q4k_device.hpp"

namespace q4k {

// Four activations at element offset `off` of a buffer (kOob: zeros).
template <bool BF16>
__device__ __forceinline__ float4 load_x4(rsrc_t r, uint32_t off) {
  if constexpr (BF16) {
    const uint2 raw = buf_load8(r, off == kOob ? kOob : 2u * off);
    return make_float4(bf16_bits_to_float(raw.x & 0xFFFFu), bf16_bits_to_float(raw.x >> 16),
                       bf16_bits_to_float(raw.y & 0xFFFFu), bf16_bits_to_float(raw.y >> 16));
  } else {
    const uint4 raw = buf_load16(r, off == kOob ? kOob : 4u * off);
    return make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                       __uint_as_float(raw.w));
  }
}

// What a lane streams per row: the 16-byte header of its block (the four
// lanes of a block load the same 16 bytes, one cache line) and quant bytes
// 32g .. 32g+31 of its quarter g.
struct RawSlice {
  uint4 h;       // d | dmin << 16, scales[0..3], scales[4..7], scales[8..11]
  uint4 q0, q1;  // quant bytes 32g .. 32g+31
};

// Block at byte offset `off` of the resource; qoff = 16 + 32g.  An offset at
// or past the resource's size reads zeros (no memory request).
__device__ __forceinline__ void load_slice(rsrc_t r, uint32_t off, uint32_t qoff, RawSlice& s) {
  s.h = buf_load16(r, off);
  s.q0 = buf_load16(r, off + qoff);
  s.q1 = buf_load16(r, off + qoff + 16u);
}

// Sum over aligned segments of SEG lanes (SEG a power of two <= 64); the
// total lands in the last lane of each segment.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v) {
  if constexpr (SEG >= 2) v += dpp_f<0xB1>(v);        // quad_perm(1,0,3,2)
  if constexpr (SEG >= 4) v += dpp_f<0x4E>(v);        // quad_perm(2,3,0,1)
  if constexpr (SEG >= 8) v += dpp_f<0x114>(v);       // row_shr:4
  if constexpr (SEG >= 16) v += dpp_f<0x118>(v);      // row_shr:8
  if constexpr (SEG >= 32) v += dpp_f<0x142, 0xA>(v); // row_bcast:15 into rows 1, 3
  if constexpr (SEG >= 64) v += dpp_f<0x143, 0xC>(v); // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ float segment_sum_rt(float v, int seg) {
  switch (seg) {
    case 1: return v;
    case 2: return segment_sum<2>(v);
    case 4: return segment_sum<4>(v);
    case 8: return segment_sum<8>(v);
    case 16: return segment_sum<16>(v);
    case 32: return segment_sum<32>(v);
    default: return segment_sum<64>(v);
  }
}

// Per-lane byte selectors that gather the 6-bit (scale, min) fields of
// sub-blocks 2g and 2g+1 from the header without a branch.  With u = 2g mod 4
// (the byte of sub-block 2g within a scale word):
//   P = [scales[u], scales[u+1], scales[u+4], scales[u+5]]  (v_perm of words 1, 2)
//   lower quarters (g < 2): the fields are the low 6 bits of P's bytes;
//   upper quarters (g >= 2): their low 4 bits are the nibbles of scales[u+8]
//   and scales[u+9] (scale: low nibble, min: high nibble; Q gathers the two
//   bytes twice) and their top 2 bits the top 2 bits of P's bytes.
struct FieldSel {
  uint32_t psel;   // v_perm selector of P from (scales[4..7] : scales[0..3])
  uint32_t qsel;   // v_perm selector of Q from (scales[8..11] : P): P itself below
  uint32_t sh_hi;  // 0 below, 2 above: bits 4-5 (below) or 6-7 (above) of P to 4-5
  uint32_t sh_m;   // 0 below, 4 above: where the mins' low 4 bits sit in Q
};

__device__ __forceinline__ FieldSel field_sel(int g) {
  const uint32_t u = (2u * static_cast<uint32_t>(g)) & 3u;
  const bool upper = g >= 2;
  FieldSel f;
  f.psel = u | (u + 1u) << 8 | (u + 4u) << 16 | (u + 5u) << 24;
  f.qsel = upper ? ((u + 4u) | (u + 5u) << 8 | (u + 4u) << 16 | (u + 5u) << 24) : 0x03020100u;
  f.sh_hi = upper ? 2u : 0u;
  f.sh_m = upper ? 4u : 0u;
  return f;
}

// The four 6-bit fields of a lane's two sub-blocks as bytes [sc0, sc1, m0, m1].
__device__ __forceinline__ uint32_t slice_fields(const uint4& h, const FieldSel& f) {
  const uint32_t P = __builtin_amdgcn_perm(h.z, h.y, f.psel);
  const uint32_t Q = __builtin_amdgcn_perm(h.w, P, f.qsel);
  const uint32_t lo = (Q & 0x00000F0Fu) | ((Q >> f.sh_m) & 0x0F0F0000u);
  return lo | ((P >> f.sh_hi) & 0x30303030u);
}

// A lane's slice of the activations in integer form.
struct XSlice {
  uint32_t dg[3][16];  // planes u0, u1 (unsigned), u2 - 64 (signed); word i holds values 4i .. 4i+3
  float scale;         // 2^(e-21) (NaN when the slice holds a non-finite value)
  float sum0, sum1;    // f32 sums of values 0..31 and 32..63
};

// sum over one 32-weight sub-block of q * a, exact in int32: |sum| <= 32*15*(2^21+1)
__device__ __forceinline__ int plane_dot(const uint32_t (&w)[8], int shift, const XSlice& x, int base) {
  uint32_t s0 = 0u, s1 = 0u;
  int s2 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = (w[i] >> shift) & 0x0F0F0F0Fu;
    s0 = __builtin_amdgcn_udot4(q, x.dg[0][base + i], s0, false);
    s1 = __builtin_amdgcn_udot4(q, x.dg[1][base + i], s1, false);
    s2 = __builtin_amdgcn_sdot4(static_cast<int>(q), static_cast<int>(x.dg[2][base + i]), s2, false);
  }
  return static_cast<int>(s0 + (s1 << 8)) + s2 * 65536;
}

// The lane's share of a row: sub-blocks 2g (low nibbles) and 2g+1 (high
// nibbles) against its slice of x,
//   d * 2^(e-21) * (sc0 * P_lo + sc1 * P_hi) - dmin * (m0 * X0 + m1 * X1).
// A lane whose loads were out of range (zeros) gives 0.
__device__ __forceinline__ float slice_dot(const RawSlice& s, const FieldSel& f, const XSlice& x) {
  const uint32_t F = slice_fields(s.h, f);
  const float d = half_bits_to_float(s.h.x & 0xFFFFu);
  const float dmin = half_bits_to_float(s.h.x >> 16);
  const uint32_t w[8] = {s.q0.x, s.q0.y, s.q0.z, s.q0.w, s.q1.x, s.q1.y, s.q1.z, s.q1.w};
  const float lo = static_cast<float>(plane_dot(w, 0, x, 0));  // sub-block 2g: low nibbles
  const float hi = static_cast<float>(plane_dot(w, 4, x, 8));  // sub-block 2g+1: high nibbles
  const float sc0 = static_cast<float>(F & 0xFFu), sc1 = static_cast<float>((F >> 8) & 0xFFu);
  const float m0 = static_cast<float>((F >> 16) & 0xFFu), m1 = static_cast<float>(F >> 24);
  const float qa = fmaf(sc1, hi, sc0 * lo);
  const float ma = fmaf(m1, x.sum1, m0 * x.sum0);
  return fmaf(qa, d * x.scale, -(dmin * ma));
}

// LDS words: the digits as twelve planes (plane 4d + j holds words 4j .. 4j+3
// of digit plane d of every slice, 16 bytes per slice, so that the lanes of
// a wavefront read consecutive 16-byte words without bank conflicts; each
// plane is padded by 16 bytes so that the four writers of a slice hit
// different banks), then the slice info [S][4] (scale, sum0, sum1, unused),
// then the row partials when a row spans wavefronts.
__host__ __device__ __forceinline__ size_t dig_plane_words(int slices) { return 4 * static_cast<size_t>(slices) + 4; }
__host__ __device__ __forceinline__ size_t xinfo_offset(int slices) { return 12 * dig_plane_words(slices); }
__host__ __device__ __forceinline__ size_t x_words(int slices) {
  return xinfo_offset(slices) + 4 * static_cast<size_t>(slices);
}

// The lane's slice of the digits from LDS.
__device__ __forceinline__ void read_digits(const uint32_t* __restrict__ dig, int S, int slice,
                                            uint32_t (&dg)[3][16]) {
  const size_t ps = dig_plane_words(S);
#pragma unroll
  for (int d = 0; d < 3; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t4 = *reinterpret_cast<const uint4*>(dig + (4 * d + i) * ps + 4 * static_cast<size_t>(slice));
      dg[d][4 * i] = t4.x; dg[d][4 * i + 1] = t4.y;
      dg[d][4 * i + 2] = t4.z; dg[d][4 * i + 3] = t4.w;
    }
}

// Converts one 16-value activation unit u (values 16u .. 16u+15, quarter u & 3
// of slice u >> 2) to byte planes in LDS.  The four units of a slice are an
// aligned lane quad, so the slice maximum and the half sums are quad DPP
// reductions; every lane of the quad must execute this (uniform control flow).
__device__ __forceinline__ void convert_unit(const float4 (&xr)[4], int u, bool valid, int S,
                                             uint32_t* __restrict__ dig, float* __restrict__ xinfo) {
  float v[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[4 * c] = xr[c].x; v[4 * c + 1] = xr[c].y; v[4 * c + 2] = xr[c].z; v[4 * c + 3] = xr[c].w;
  }
  float amax = 0.f, sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = fmaxf(amax, fabsf(v[i]));
    sum += v[i];
  }
  amax = fmaxf(amax, dpp_f<0xB1>(amax));
  amax = fmaxf(amax, dpp_f<0x4E>(amax));
  sum += dpp_f<0xB1>(sum);  // units 0+1 and 2+3: the two 32-value halves
  // |x| < 2^e over the slice; e >= -105 keeps 2^(21-e) a normal f32 (slices
  // below 2^-106 keep fewer bits), and an all-zero slice takes e = 0
  const int eb = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = amax > 0.f ? max(eb - 126, -105) : 0;
  if (!valid) return;
  const float mul = __uint_as_float(static_cast<uint32_t>(127 + 21 - e) << 23);  // 2^(21-e)
  uint32_t p0[4], p1[4], p2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = __float_as_uint(fmaf(v[4 * q + r], mul, 12582912.0f));
    // byte transpose: t01 = [f0.b0 f1.b0 f0.b1 f1.b1], t23 likewise
    const uint32_t t01 = __builtin_amdgcn_perm(f[1], f[0], 0x05010400u);
    const uint32_t t23 = __builtin_amdgcn_perm(f[3], f[2], 0x05010400u);
    p0[q] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    p1[q] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    const uint32_t h = __builtin_amdgcn_perm(f[1], f[0], 0x0C0C0602u) |
                       __builtin_amdgcn_perm(f[3], f[2], 0x06020C0Cu);  // the u2 bytes (32..96)
    p2[q] = (h + 0x40404040u) ^ 0x80808080u;  // bytewise u2 - 64 (no carries: u2 + 64 < 256)
  }
  const int s = u >> 2, qq = u & 3;
  const size_t ps = dig_plane_words(S);
  uint32_t* base = dig + qq * ps + 4 * static_cast<size_t>(s);
  *reinterpret_cast<uint4*>(base) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
  *reinterpret_cast<uint4*>(base + 4 * ps) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
  *reinterpret_cast<uint4*>(base + 8 * ps) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
  if (qq == 0) {
    // amax - amax is 0 for a finite maximum and NaN otherwise
    xinfo[4 * s] = __uint_as_float(static_cast<uint32_t>(127 - 21 + e) << 23) + (amax - amax);
    xinfo[4 * s + 1] = sum;
  } else if (qq == 2) {
    xinfo[4 * s + 2] = sum;
  }
}

}  // namespace q4k
