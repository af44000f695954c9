// Q6_K decode GEMV (one token, f32 activations), gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q6k_gemv_cached_async: the Q4_K
// GEMV's counterpart for Q6_K weights, used for the LM head: y[j] = sum_i
// w[j][i] * x[i] with f32 x of length k and f32 y of length n.  The page
// names the format only; the layout read here is GGML's block_q6_K (256
// weights in 210 bytes): ql[128] the low 4 bits, qh[64] the high 2 bits,
// scales[16] signed 8-bit (one per 16 weights), d binary16.  Weight
// 128h + 32r + l (h the half, r its quarter, l < 32) takes the low nibble
// (r < 2) or high nibble (r >= 2) of ql[64h + 32(r & 1) + l] and bits 2r, 2r+1
// of qh[32h + l]; with u that 6-bit value, w = d * scales[i / 16] * (u - 32).
//
// Layout.  A row is cut into 4*(k/256) slices of 64 weights: slice (h, s) of
// a block holds quarters r = s and r = s + 2 of half h, i.e. both nibbles of
// ql[64h + 32s .. +31] and the matching bit pairs of qh[32h .. 32h+31].  Each
// lane owns one slice position for the whole kernel and keeps its 64 x values
// in registers with the sum of x over each of its four 16-weight sub-blocks,
// so sum (u - 32) x = sum u x - 32 sum x and the 6-bit values go to f32
// straight from their bytes (v_cvt_f32_ubyte).  A block starts at a multiple
// of 210 bytes, i.e. only 2-byte aligned: a lane loads the aligned dwords
// around its fields (nine for 32 bytes, the ninth only when the block is not
// dword-aligned, so no load reaches past the block) and shifts them into place
// with v_alignbyte; d comes from a 16-bit load.  A wavefront covers 16
// consecutive blocks of a row; wider rows span several wavefronts, whose sums
// meet in LDS.  PF rows are in flight per wavefront; the reduction order is
// fixed (deterministic).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kQ6Threads = 512;
constexpr int kQ6BlockBytes = 210;
constexpr int kQ6PF = 4;
constexpr int kQ6MaxRowsPerGroup = 256;

struct Q6Geo {
  int wr;   // wavefronts per row
  int rs;   // row slots per workgroup
  int rpg;  // rows per workgroup (a multiple of rs)
};

struct Q6Raw {
  uint4 l0, l1;     // ql window, dwords 0-7
  uint32_t l2;      // ql window, dword 8
  uint4 h0, h1;     // qh window
  uint32_t h2;
  uint2 s01;        // scale window (8 bytes of this half's scales), dwords 0-1
  uint32_t s2;
  uint32_t d;       // binary16 bits of d
};

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
}

__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0);
}

// a: byte offset of the block within the resource (kOob for no row);
// h, s: the lane's slice of the block
__device__ __forceinline__ void load_q6(rsrc_t r, uint32_t a, int h, int s, Q6Raw& raw) {
  const bool none = a == kOob;
  const uint32_t sh = a & 3u;
  const uint32_t ql = none ? kOob : (a + 64u * h + 32u * s) & ~3u;
  const uint32_t qh = none ? kOob : (a + 128u + 32u * h) & ~3u;
  const uint32_t sc = none ? kOob : (a + 192u + 8u * h) & ~3u;
  raw.l0 = buf_load16(r, ql);
  raw.l1 = buf_load16(r, none ? kOob : ql + 16u);
  raw.l2 = buf_load4(r, none || sh == 0 ? kOob : ql + 32u);
  raw.h0 = buf_load16(r, qh);
  raw.h1 = buf_load16(r, none ? kOob : qh + 16u);
  raw.h2 = buf_load4(r, none || sh == 0 ? kOob : qh + 32u);
  raw.s01 = buf_load8(r, sc);
  raw.s2 = buf_load4(r, none || sh == 0 ? kOob : sc + 8u);
  raw.d = buf_load2(r, none ? kOob : a + 208u);
}

// Lane permute on the VALU (DPP); lanes whose source is out of range read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_q6(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, true));
}

// Sum over the 64 lanes, landing in lane 63.
__device__ __forceinline__ float total_in_last_lane(float v) {
  v += dpp_q6<0xB1>(v);        // quad_perm(1,0,3,2)
  v += dpp_q6<0x4E>(v);        // quad_perm(2,3,0,1)
  v += dpp_q6<0x114>(v);       // row_shr:4
  v += dpp_q6<0x118>(v);       // row_shr:8
  v += dpp_q6<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_q6<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// signed byte e of w as a float (v_bfe_i32; the builtin's result type is
// unsigned, so it goes back to int before the conversion)
__device__ __forceinline__ float scale_at(uint32_t w, int e) {
  return static_cast<float>(static_cast<int>(__builtin_amdgcn_sbfe(w, 8 * e, 8)));
}

__device__ __forceinline__ float byte_f(uint32_t w, int e) {
  return static_cast<float>((w >> (8 * e)) & 0xFFu);  // v_cvt_f32_ubyte<e>
}

__global__ __launch_bounds__(kQ6Threads) void q6k_gemv_kernel(const uint8_t* __restrict__ w,
                                                              const float* __restrict__ x,
                                                              float* __restrict__ y, int n, int k,
                                                              Q6Geo geo) {
  extern __shared__ __attribute__((aligned(16))) float part[];  // [rpg][wr]
  const int K = k >> 8;
  const int S = 4 * K;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / geo.wr;  // uniform
  const int wpart = wave - slot * geo.wr;
  const int slice = wpart * 64 + lane;
  const bool lane_ok = slice < S;
  const int b = lane_ok ? slice >> 2 : 0;
  const int h = (slice >> 1) & 1;
  const int s = slice & 1;

  // 1. this lane's x: quarter s (xl) and quarter s + 2 (xh) of half h of
  //    block b, and their sums over each 16-value sub-block
  const rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(k) * 4u);
  float xl[32], xh[32];
  {
    const uint32_t lo = lane_ok ? (256u * b + 128u * h + 32u * s) * 4u : kOob;
    const uint32_t hi = lane_ok ? lo + 64u * 4u : kOob;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 vl = buf_load16(rx, lo == kOob ? kOob : lo + 16u * c);
      const uint4 vh = buf_load16(rx, hi == kOob ? kOob : hi + 16u * c);
      xl[4 * c] = __uint_as_float(vl.x);
      xl[4 * c + 1] = __uint_as_float(vl.y);
      xl[4 * c + 2] = __uint_as_float(vl.z);
      xl[4 * c + 3] = __uint_as_float(vl.w);
      xh[4 * c] = __uint_as_float(vh.x);
      xh[4 * c + 1] = __uint_as_float(vh.y);
      xh[4 * c + 2] = __uint_as_float(vh.z);
      xh[4 * c + 3] = __uint_as_float(vh.w);
    }
  }
  float sxl0 = 0.f, sxl1 = 0.f, sxh0 = 0.f, sxh1 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sxl0 += xl[i];
    sxl1 += xl[16 + i];
    sxh0 += xh[i];
    sxh1 += xh[16 + i];
  }

  // 2. the workgroup's rows: slot `slot` takes rows slot, slot + rs, ...  The
  //    resource starts at the 16-byte boundary at or below the first row.
  const int row0 = blockIdx.x * geo.rpg;
  const int rows = min(geo.rpg, n - row0);
  const uint32_t rowbytes = static_cast<uint32_t>(K) * kQ6BlockBytes;
  const size_t first = static_cast<size_t>(row0) * rowbytes;
  const uint32_t delta = static_cast<uint32_t>(first & 15u);
  const rsrc_t rw = make_rsrc(w + (first - delta), delta + static_cast<uint32_t>(rows) * rowbytes);
  const uint32_t stride = static_cast<uint32_t>(geo.rs) * rowbytes;
  const uint32_t base = delta + static_cast<uint32_t>(slot) * rowbytes + static_cast<uint32_t>(b) * kQ6BlockBytes;
  const int nit = (rows - slot + geo.rs - 1) / geo.rs;  // rows of this slot (uniform)
  auto row_off = [&](int it) -> uint32_t {
    return lane_ok && it < nit ? base + static_cast<uint32_t>(it) * stride : kOob;
  };
  const int groups = (nit + kQ6PF - 1) / kQ6PF;
  const uint32_t qh_shift = 2u * static_cast<uint32_t>(s);

  Q6Raw raw[kQ6PF];
#pragma unroll
  for (int p = 0; p < kQ6PF; ++p) load_q6(rw, row_off(p), h, s, raw[p]);

  for (int grp = 0; grp < groups; ++grp) {
#pragma unroll
    for (int p = 0; p < kQ6PF; ++p) {
      const int it = grp * kQ6PF + p;
      const uint32_t sh = row_off(it) & 3u;  // 0 or 2: the block's offset within its dword
      const Q6Raw cur = raw[p];
      // the next row of this register set is in flight while this one is used
      load_q6(rw, row_off(it + kQ6PF), h, s, raw[p]);
      const uint32_t lw[9] = {cur.l0.x, cur.l0.y, cur.l0.z, cur.l0.w, cur.l1.x, cur.l1.y, cur.l1.z, cur.l1.w, cur.l2};
      const uint32_t hw[9] = {cur.h0.x, cur.h0.y, cur.h0.z, cur.h0.w, cur.h1.x, cur.h1.y, cur.h1.z, cur.h1.w, cur.h2};
      float al0 = 0.f, al1 = 0.f, ah0 = 0.f, ah1 = 0.f;  // sum u x per sub-block
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t qlw = __builtin_amdgcn_alignbyte(lw[j + 1], lw[j], sh);
        const uint32_t qhw = __builtin_amdgcn_alignbyte(hw[j + 1], hw[j], sh) >> qh_shift;
        const uint32_t ulo = (qlw & 0x0F0F0F0Fu) | ((qhw & 0x03030303u) << 4);
        const uint32_t uhi = ((qlw >> 4) & 0x0F0F0F0Fu) | (((qhw >> 4) & 0x03030303u) << 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j < 4) {
            al0 = fmaf(byte_f(ulo, e), xl[4 * j + e], al0);
            ah0 = fmaf(byte_f(uhi, e), xh[4 * j + e], ah0);
          } else {
            al1 = fmaf(byte_f(ulo, e), xl[4 * j + e], al1);
            ah1 = fmaf(byte_f(uhi, e), xh[4 * j + e], ah1);
          }
        }
      }
      // scales 8h .. 8h+7 of the block; the lane's are 2s, 2s+1 (quarter s)
      // and 2s+4, 2s+5 (quarter s + 2)
      const uint32_t sc0 = __builtin_amdgcn_alignbyte(cur.s01.y, cur.s01.x, sh);
      const uint32_t sc1 = __builtin_amdgcn_alignbyte(cur.s2, cur.s01.y, sh);
      const float fl0 = scale_at(sc0, 2 * s), fl1 = scale_at(sc0, 2 * s + 1);
      const float fh0 = scale_at(sc1, 2 * s), fh1 = scale_at(sc1, 2 * s + 1);
      float v = fl0 * fmaf(-32.f, sxl0, al0);
      v = fmaf(fl1, fmaf(-32.f, sxl1, al1), v);
      v = fmaf(fh0, fmaf(-32.f, sxh0, ah0), v);
      v = fmaf(fh1, fmaf(-32.f, sxh1, ah1), v);
      v *= half_bits_to_float(cur.d & 0xFFFFu);
      const float tot = total_in_last_lane(lane_ok ? v : 0.f);
      if (it < nit && lane == 63) {
        const int r = slot + it * geo.rs;
        if (geo.wr == 1)
          y[row0 + r] = tot;
        else
          part[r * geo.wr + wpart] = tot;
      }
    }
  }
  if (geo.wr > 1) {
    __syncthreads();
    for (int r = tid; r < rows; r += blockDim.x) {
      float acc = 0.f;
      for (int q = 0; q < geo.wr; ++q) acc += part[r * geo.wr + q];
      y[row0 + r] = acc;
    }
  }
}

Q6Geo make_q6_geo(int n, int k) {
  Q6Geo g{};
  const int S = 4 * (k / kQK);
  g.wr = (S + 63) / 64;
  g.rs = g.wr >= 4 ? 1 : (4 + g.wr - 1) / g.wr;
  // about two workgroups per compute unit (512), whole slots
  long long want = (static_cast<long long>(n) + 511) / 512;
  if (want < g.rs) want = g.rs;
  if (want > kQ6MaxRowsPerGroup) want = kQ6MaxRowsPerGroup;
  g.rpg = static_cast<int>((want + g.rs - 1) / g.rs * g.rs);
  return g;
}

}  // namespace

hipError_t launch_q6k_gemv(const uint8_t* w, const float* x, float* y, int n, int k, hipStream_t stream) {
  if (k < kQK || k % kQK || k > 32768 || n < 1) return hipErrorInvalidValue;
  const Q6Geo g = make_q6_geo(n, k);
  // every offset into a workgroup's rows stays below 2^31
  if (static_cast<long long>(g.rpg) * (k / kQK) * kQ6BlockBytes + 16 >= (1LL << 31)) return hipErrorInvalidValue;
  const size_t lds = g.wr > 1 ? static_cast<size_t>(g.rpg) * g.wr * sizeof(float) : 0;
  const dim3 grid((n + g.rpg - 1) / g.rpg);
  q6k_gemv_kernel<<<grid, dim3(64 * g.wr * g.rs), lds, stream>>>(w, x, y, n, k, g);
  return hipGetLastError();
}

}  // namespace q4k
