// Load-time Q4_K weight quantiser, gfx950.
//
// "spark_model/layers/ops/q4k_mmq.rs", quantize_weight_q4k: weights are
// encoded to GGML block_q4_K at load time; the pages print no algorithm.
// The fit used here, every step in binary32 with round-to-nearest-even, per
// 32-value sub-block j of a 256-value block:
//   lo = min(0, min x), hi = max x, o = 0 - lo, s = hi > lo ? (hi - lo)/15 : 0
//   d = binary16(max_j s / 63), dmin = binary16(max_j o / 63)   (saturating)
//   sc_j = rint(s_j / d), m_j = rint(o_j / dmin)   clamped to 0..63 (0 for a 0 divisor)
//   q = rint((x + dmin*m_j) / (d*sc_j))           clamped to 0..15 (0 for a 0 step)
// so d*sc_j*q - dmin*m_j is the nearest point of the block's grid.  Every
// operation is an IEEE binary32 operation (min, max, subtract, correctly
// rounded divide, rint, exact products), so the bytes are reproducible.
//
// Four blocks per wavefront, one per 16-lane row: lane l of a row holds
// values 16l .. 16l+15 of its block (sub-block l/2).  Sub-block extrema take
// one register-level lane exchange (DPP) and the block maxima three more, all
// within the row, so no exchange goes through the LDS or crosses into another
// block; lane l with l % 4 < 2 packs its sixteen quants with the sixteen of
// lane l + 2 (the high nibbles of the same bytes) into 16 bytes of the quant
// field, and lanes 0, 16, 32 and 48 write the headers.  Its vector-ALU work
// (the per-sub-block divisions, the codes, the header gathering) and latency
// bound it rather than the bytes it reads (4 or 2 per value) and writes
// (0.5625 per value).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kQzThreads = 256;  // sixteen blocks per workgroup, four per wavefront

// DPP move of v (row_mask all rows); lanes outside BANKS (4-lane groups of a
// 16-lane row) keep old
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_move(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL, 0xF,
                                                               BANKS, false));
}

// v of lane ^ 1, ^ 2, ^ 4 and ^ 8
__device__ __forceinline__ float lane_xor1(float v) { return dpp_move<0xB1, 0xF>(v, v); }  // quad_perm(1,0,3,2)
__device__ __forceinline__ float lane_xor2(float v) { return dpp_move<0x4E, 0xF>(v, v); }  // quad_perm(2,3,0,1)
__device__ __forceinline__ float lane_xor4(float v) {
  const float t = dpp_move<0x104, 0x5>(v, v);  // row_shl:4 into lanes 0-3 and 8-11 of a row
  return dpp_move<0x114, 0xA>(t, v);           // row_shr:4 into lanes 4-7 and 12-15
}
__device__ __forceinline__ float lane_xor8(float v) { return dpp_move<0x128, 0xF>(v, v); }  // row_ror:8

__device__ __forceinline__ uint32_t lane_xor2_u(uint32_t v) {
  return __float_as_uint(lane_xor2(__uint_as_float(v)));
}

// binary16 bits of v >= 0 (nearest even), 65504 where the rounding would overflow
__device__ __forceinline__ uint32_t f16_bits_saturating(float v) {
  return v >= 65520.0f ? 0x7BFFu : float_to_half_bits(v);
}

template <bool BF16>
__global__ __launch_bounds__(kQzThreads) void quantize_q4k_kernel(const void* __restrict__ x,
                                                                  uint8_t* __restrict__ w,
                                                                  long long nblocks) {
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15;  // lane within the block's row
  const long long blk = (static_cast<long long>(blockIdx.x) * (kQzThreads / 64) + (threadIdx.x >> 6)) * 4 +
                        (lane >> 4);
  const bool valid = blk < nblocks;  // a missing block reads block 0 and stores nothing
  // rows are contiguous and a whole number of blocks long, so block blk holds
  // values 256 blk .. 256 blk + 255 of the matrix
  const size_t e = static_cast<size_t>(valid ? blk : 0) * kQK + 16 * rl;
  float v[16];
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e + 8 * c);
      const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = bf16_bits_to_float(r4[i] & 0xFFFFu);
        v[8 * c + 2 * i + 1] = bf16_bits_to_float(r4[i] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e + 4 * c);
      v[4 * c] = f.x;
      v[4 * c + 1] = f.y;
      v[4 * c + 2] = f.z;
      v[4 * c + 3] = f.w;
    }
  }

  // sub-block extrema over its 2 lanes, then the step and offset
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  mn = fminf(mn, lane_xor1(mn));
  mx = fmaxf(mx, lane_xor1(mx));
  const float lo = fminf(mn, 0.0f);
  const float o = 0.0f - lo;
  const float s = mx > lo ? (mx - lo) / 15.0f : 0.0f;

  // block scale and min: maxima over the 8 sub-blocks (lanes l ^ 2, ^ 4, ^ 8)
  float smax = fmaxf(s, lane_xor2(s));
  float omax = fmaxf(o, lane_xor2(o));
  smax = fmaxf(smax, lane_xor4(smax));
  omax = fmaxf(omax, lane_xor4(omax));
  smax = fmaxf(smax, lane_xor8(smax));
  omax = fmaxf(omax, lane_xor8(omax));
  const uint32_t dbits = f16_bits_saturating(smax / 63.0f);
  const uint32_t mbits = f16_bits_saturating(omax / 63.0f);
  const float d = half_bits_to_float(dbits);
  const float dmin = half_bits_to_float(mbits);
  const int sc = d > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(s / d), 0.0f), 63.0f)) : 0;
  const int mm = dmin > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(o / dmin), 0.0f), 63.0f)) : 0;
  const float ds = d * static_cast<float>(sc);    // exact: 11 x 6 bits
  const float dm = dmin * static_cast<float>(mm);

  // quants: value 16l + i of the block is nibble (l % 4 < 2 ? low : high) of
  // quant byte 32 (l / 4) + 16 (l % 2) + i.  The code is rint of the
  // correctly rounded quotient t = (x + dm) / ds.  Fast path: p = (x + dm) *
  // rcp(ds) with v_rcp_f32 (1 ulp) is within 1.6 * 2^-23 |t| of t, and
  // binary32 t within 2^-24 |t|: where |t| <= 16.5 matters, less than
  // 4.2 * 2^-20 apart.  When p is more than 2^-17 from every half-integer,
  // both round to the same integer; otherwise (ties and near-ties, rare in
  // real weights) the wavefront takes the exact division.
  uint32_t q4[4] = {0u, 0u, 0u, 0u};
  {
    const float inv = ds > 0.0f ? __builtin_amdgcn_rcpf(ds) : 0.0f;
    bool near_tie = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = (v[i] + dm) * inv;
      const float r = rintf(p);
      near_tie |= fabsf(fabsf(p - r) - 0.5f) <= 0x1p-17f;
      const uint32_t q = static_cast<uint32_t>(fminf(fmaxf(r, 0.0f), 15.0f));
      q4[i >> 2] |= q << (8 * (i & 3));
    }
    if (__any(near_tie)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) q4[c] = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t q =
            ds > 0.0f ? static_cast<uint32_t>(fminf(fmaxf(rintf((v[i] + dm) / ds), 0.0f), 15.0f)) : 0u;
        q4[i >> 2] |= q << (8 * (i & 3));
      }
    }
  }
  uint32_t hi[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) hi[c] = lane_xor2_u(q4[c]);
  uint8_t* out = w + static_cast<size_t>(valid ? blk : 0) * kBlockBytes;
  if (valid && (rl & 2) == 0)
    *reinterpret_cast<uint4*>(out + 16 + 32 * (rl >> 2) + 16 * (rl & 1)) =
        make_uint4(q4[0] | (hi[0] << 4), q4[1] | (hi[1] << 4), q4[2] | (hi[2] << 4), q4[3] | (hi[3] << 4));

  // headers: d, dmin and the eight 6-bit pairs of each block (sub-block j's
  // in lane 2j of the block's row)
  uint32_t hw[4][3];
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    uint32_t scj[8], mj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      scj[j] = static_cast<uint32_t>(__builtin_amdgcn_readlane(sc, 16 * row + 2 * j));
      mj[j] = static_cast<uint32_t>(__builtin_amdgcn_readlane(mm, 16 * row + 2 * j));
    }
    hw[row][0] = hw[row][1] = hw[row][2] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b0 = (scj[j] & 63u) | ((scj[j + 4] >> 4) << 6);
      const uint32_t b1 = (mj[j] & 63u) | ((mj[j + 4] >> 4) << 6);
      const uint32_t b2 = (scj[j + 4] & 15u) | ((mj[j + 4] & 15u) << 4);
      hw[row][0] |= b0 << (8 * j);
      hw[row][1] |= b1 << (8 * j);
      hw[row][2] |= b2 << (8 * j);
    }
  }
  if (valid && rl == 0) {
    const int row = lane >> 4;
    uint32_t h0 = hw[0][0], h1 = hw[0][1], h2 = hw[0][2];
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (row == r) {
        h0 = hw[r][0];
        h1 = hw[r][1];
        h2 = hw[r][2];
      }
    *reinterpret_cast<uint4*>(out) = make_uint4(dbits | (mbits << 16), h0, h1, h2);
  }
}

}  // namespace

hipError_t launch_quantize_q4k(const void* x, int x_bf16, int rows, int cols, uint8_t* w,
                               hipStream_t stream) {
  if (rows < 1 || cols < kQK || cols % kQK) return hipErrorInvalidValue;
  const long long nblocks = static_cast<long long>(rows) * (cols / kQK);
  constexpr int per_group = 4 * (kQzThreads / 64);
  const long long groups = (nblocks + per_group - 1) / per_group;
  if (groups > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups));
  if (x_bf16)
    quantize_q4k_kernel<true><<<grid, dim3(kQzThreads), 0, stream>>>(x, w, nblocks);
  else
    quantize_q4k_kernel<false><<<grid, dim3(kQzThreads), 0, stream>>>(x, w, nblocks);
  return hipGetLastError();
}

}  // namespace q4k
