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
// One wavefront per block: lane l holds values 4l .. 4l+3 (sub-block l/8).
// Sub-block extrema take three register-level lane exchanges among its 8 lanes
// (DPP) and the block maxima three more (DPP and the gfx950 row/half swaps), so
// no exchange goes through the LDS; lane l < 8 of each 16 packs its four quants with
// the four of lane l+8 (the high nibbles, sub-block 2g+1) into one word of
// the quant field, and lane 0 writes the header.  The kernel is bound by the
// bytes it reads (4 or 2 per value) and writes (0.5625 per value).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kQzThreads = 256;  // four blocks per workgroup, one per wavefront

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

// maximum of v over lanes l, l ^ 16, l ^ 32, l ^ 48: a row swap and a half
// swap of two copies put each partner's value beside the lane's own
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
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
  const long long blk = static_cast<long long>(blockIdx.x) * (kQzThreads / 64) + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // whole wavefronts; the kernel has no barrier
  // rows are contiguous and a whole number of blocks long, so block blk holds
  // values 256 blk .. 256 blk + 255 of the matrix
  const size_t e = static_cast<size_t>(blk) * kQK + 4 * lane;
  float v[4];
  if constexpr (BF16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + e);
    v[0] = bf16_bits_to_float(raw.x & 0xFFFFu);
    v[1] = bf16_bits_to_float(raw.x >> 16);
    v[2] = bf16_bits_to_float(raw.y & 0xFFFFu);
    v[3] = bf16_bits_to_float(raw.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }

  // sub-block extrema over its 8 lanes, then the step and offset
  float mn = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
  float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  mn = fminf(mn, lane_xor1(mn));
  mx = fmaxf(mx, lane_xor1(mx));
  mn = fminf(mn, lane_xor2(mn));
  mx = fmaxf(mx, lane_xor2(mx));
  mn = fminf(mn, lane_xor4(mn));
  mx = fmaxf(mx, lane_xor4(mx));
  const float lo = fminf(mn, 0.0f);
  const float o = 0.0f - lo;
  const float s = mx > lo ? (mx - lo) / 15.0f : 0.0f;

  // block scale and min
  const float smax = max_xor16_32(fmaxf(s, lane_xor8(s)));
  const float omax = max_xor16_32(fmaxf(o, lane_xor8(o)));
  const uint32_t dbits = f16_bits_saturating(smax / 63.0f);
  const uint32_t mbits = f16_bits_saturating(omax / 63.0f);
  const float d = half_bits_to_float(dbits);
  const float dmin = half_bits_to_float(mbits);
  const int sc = d > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(s / d), 0.0f), 63.0f)) : 0;
  const int mm = dmin > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(o / dmin), 0.0f), 63.0f)) : 0;
  const float ds = d * static_cast<float>(sc);    // exact: 11 x 6 bits
  const float dm = dmin * static_cast<float>(mm);

  // quants, packed with the partner lane's high nibbles
  uint32_t qw = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t q = ds > 0.0f ? static_cast<uint32_t>(fminf(fmaxf(rintf((v[r] + dm) / ds), 0.0f), 15.0f)) : 0u;
    qw |= q << (8 * r);
  }
  const uint32_t hiw = __float_as_uint(lane_xor8(__uint_as_float(qw)));
  uint8_t* out = w + static_cast<size_t>(blk) * kBlockBytes;
  if ((lane & 8) == 0)
    *reinterpret_cast<uint32_t*>(out + 16 + 32 * (lane >> 4) + 4 * (lane & 7)) = qw | (hiw << 4);

  // header: d, dmin and the eight 6-bit pairs (sub-block j's in lane 8j)
  uint32_t scj[8], mj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    scj[j] = static_cast<uint32_t>(__builtin_amdgcn_readlane(sc, 8 * j));
    mj[j] = static_cast<uint32_t>(__builtin_amdgcn_readlane(mm, 8 * j));
  }
  if (lane == 0) {
    uint32_t hw[3] = {0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b0 = (scj[j] & 63u) | ((scj[j + 4] >> 4) << 6);
      const uint32_t b1 = (mj[j] & 63u) | ((mj[j + 4] >> 4) << 6);
      const uint32_t b2 = (scj[j + 4] & 15u) | ((mj[j + 4] & 15u) << 4);
      hw[0] |= b0 << (8 * j);
      hw[1] |= b1 << (8 * j);
      hw[2] |= b2 << (8 * j);
    }
    *reinterpret_cast<uint4*>(out) = make_uint4(dbits | (mbits << 16), hw[0], hw[1], hw[2]);
  }
}

}  // namespace

hipError_t launch_quantize_q4k(const void* x, int x_bf16, int rows, int cols, uint8_t* w,
                               hipStream_t stream) {
  if (rows < 1 || cols < kQK || cols % kQK) return hipErrorInvalidValue;
  const long long nblocks = static_cast<long long>(rows) * (cols / kQK);
  const long long groups = (nblocks + kQzThreads / 64 - 1) / (kQzThreads / 64);
  if (groups > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(groups));
  if (x_bf16)
    quantize_q4k_kernel<true><<<grid, dim3(kQzThreads), 0, stream>>>(x, w, nblocks);
  else
    quantize_q4k_kernel<false><<<grid, dim3(kQzThreads), 0, stream>>>(x, w, nblocks);
  return hipGetLastError();
}

}  // namespace q4k
