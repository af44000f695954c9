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
// lane owns one slice position for the whole kernel.  It holds its 64 x
// values once, as integers X = rint(x * 2^(21-e)) with 2^e above the slice's
// largest |x| (so within 2^-22 of that maximum), split into three byte planes
// (two unsigned, the top one signed); with the integer sum SX of X over each
// of its four 16-weight sub-blocks, a sub-block's sum (u - 32) x is
// 2^(e-21) (sum u X - 32 SX) and sum u X takes three v_dot4 per four weights
// (v_dot4_u32_u8 on the low planes, v_dot4_i32_i8 on the top one; u < 64).
//
// Loads.  A block starts at a multiple of 210 bytes, i.e. only 2-byte
// aligned: the four lanes of a block (a lane quad) load the aligned dwords
// around their fields and shift them into place with v_alignbyte.  Each lane
// loads its 32 ql bytes and 32 qh bytes (eight dwords each); the ninth dword
// a misaligned window needs is the first dword of a quad-mate's window, and
// the 16 scale bytes are one dword per lane, both passed around the quad by
// DPP.  The last dword of the block (scales 14-15 and d) or, for a
// dword-aligned block, d alone is one more load, so no load reaches past the
// block and every load instruction of a wavefront touches few cache lines.
// A wavefront covers 16 consecutive blocks of a row; wider rows span several
// wavefronts, whose sums meet in LDS.  PF rows are in flight per wavefront,
// one workgroup per compute unit (more rows in flight measured slower); the
// reduction order is fixed (deterministic).
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
  uint4 h0, h1;     // qh window, dwords 0-7
  uint32_t sd;      // dword q of the block's scale window (lane q of the quad)
  uint32_t tail4;   // misaligned block: the dword ending at the block's end
  uint32_t tail2;   // aligned block: d
};

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
}

__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0);
}

// a: byte offset of the block within the resource (kOob for no row);
// h, s: the lane's slice of the block (quad lane q = 2h + s)
__device__ __forceinline__ void load_q6(rsrc_t r, uint32_t a, int h, int s, Q6Raw& raw) {
  __builtin_amdgcn_sched_barrier(0);
  const bool none = a == kOob;
  const uint32_t sh = a & 3u;
  const uint32_t ql = none ? kOob : (a + 64u * h + 32u * s) & ~3u;
  const uint32_t qh = none ? kOob : (a + 128u + 32u * h) & ~3u;
  raw.l0 = buf_load16(r, ql);
  raw.l1 = buf_load16(r, none ? kOob : ql + 16u);
  raw.h0 = buf_load16(r, qh);
  raw.h1 = buf_load16(r, none ? kOob : qh + 16u);
  raw.sd = buf_load4(r, none ? kOob : ((a + 192u) & ~3u) + 8u * h + 4u * s);
  // misaligned block: the dword at a + 206 (scales 14-15, d); aligned: d at a + 208
  // (kept apart until the row is used: combining them here would wait for both)
  raw.tail4 = buf_load4(r, none || sh == 0 ? kOob : a + 206u);
  raw.tail2 = buf_load2(r, none || sh != 0 ? kOob : a + 208u);
  // a row's loads are issued together and rows in order: the vector memory
  // counter drains in issue order, so a row issued late would make every
  // earlier row wait for it
  __builtin_amdgcn_sched_barrier(0);
}

// v of lane SRC of this lane's quad (DPP quad_perm broadcast)
template <int SRC>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), SRC * 0x55, 0xF, 0xF, false));
}

// v of quad lane q + 1 (q = 0, 1, 2; lane 3 reads lane 0)
__device__ __forceinline__ uint32_t quad_next(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x39, 0xF, 0xF, false));
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

// x of one 64-value slice as byte planes of X = rint(x * 2^(21-e)):
// p0, p1 the low and middle bytes (unsigned), p2 the top byte (signed); four
// consecutive values per dword, values 0-31 (quarter s) in words 0-7 and
// values 32-63 (quarter s + 2) in words 8-15
struct XPlanes {
  uint32_t p0[16], p1[16], p2[16];
  int sx[4];    // sum of X over each 16-value sub-block
  float unit;   // 2^(e-21)
};

__device__ __forceinline__ void make_planes(const float (&v)[64], XPlanes& xp) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // 2^e > amax >= 2^(e-1); e = 0 for an all-zero slice
  const int e = amax > 0.f ? ilogbf(amax) + 1 : 0;
  xp.unit = ldexpf(1.f, e - 21);
#pragma unroll
  for (int q = 0; q < 4; ++q) xp.sx[q] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t b0 = 0, b1 = 0, b2 = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int X = static_cast<int>(rintf(ldexpf(v[4 * j + c], 21 - e)));  // |X| <= 2^21
      xp.sx[j / 4] += X;
      b0 |= (static_cast<uint32_t>(X) & 0xFFu) << (8 * c);
      b1 |= ((static_cast<uint32_t>(X) >> 8) & 0xFFu) << (8 * c);
      b2 |= ((static_cast<uint32_t>(X) >> 16) & 0xFFu) << (8 * c);
    }
    xp.p0[j] = b0;
    xp.p1[j] = b1;
    xp.p2[j] = b2;
  }
}

// this lane's x: quarter s (values 0-31) and quarter s + 2 (values 32-63) of
// half h of block b
__device__ __forceinline__ void load_x(rsrc_t rx, bool lane_ok, int b, int h, int s, float (&xv)[64]) {
  const uint32_t lo = lane_ok ? (256u * b + 128u * h + 32u * s) * 4u : kOob;
  const uint32_t hi = lane_ok ? lo + 64u * 4u : kOob;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 vl = buf_load16(rx, lo == kOob ? kOob : lo + 16u * c);
    const uint4 vh = buf_load16(rx, hi == kOob ? kOob : hi + 16u * c);
    xv[4 * c] = __uint_as_float(vl.x);
    xv[4 * c + 1] = __uint_as_float(vl.y);
    xv[4 * c + 2] = __uint_as_float(vl.z);
    xv[4 * c + 3] = __uint_as_float(vl.w);
    xv[32 + 4 * c] = __uint_as_float(vh.x);
    xv[32 + 4 * c + 1] = __uint_as_float(vh.y);
    xv[32 + 4 * c + 2] = __uint_as_float(vh.z);
    xv[32 + 4 * c + 3] = __uint_as_float(vh.w);
  }
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

  // The workgroup's rows: slot `slot` takes rows slot, slot + rs, ...  The
  // resource starts at the 16-byte boundary at or below the first row.
  const rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(k) * 4u);
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

  // x loads, then the first rows' loads, then the conversion of x to byte
  // planes (which waits for the x loads only)
  Q6Raw raw[kQ6PF];
  XPlanes xp;
  {
    float xv[64];
    load_x(rx, lane_ok, b, h, s, xv);
    __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the row loads
#pragma unroll
    for (int p = 0; p < kQ6PF; ++p) load_q6(rw, row_off(p), h, s, raw[p]);
    __builtin_amdgcn_sched_barrier(0);
    make_planes(xv, xp);
  }

  const float sx0 = static_cast<float>(32 * xp.sx[0]), sx1 = static_cast<float>(32 * xp.sx[1]);
  const float sx2 = static_cast<float>(32 * xp.sx[2]), sx3 = static_cast<float>(32 * xp.sx[3]);

  for (int grp = 0; grp < groups; ++grp) {
#pragma unroll
    for (int p = 0; p < kQ6PF; ++p) {
      const int it = grp * kQ6PF + p;
      const uint32_t sh = row_off(it) & 3u;  // 0 or 2: the block's offset within its dword
      const Q6Raw& cur = raw[p];
      // the ninth dwords of the ql and qh windows and the scale window, from
      // quad-mates: ql of (h, 0) continues into ql of (h, 1), ql of (0, 1)
      // into ql of (1, 0), ql of (1, 1) into qh of half 0; qh of half 0 into
      // qh of half 1, qh of half 1 into the scale window
      const uint32_t next_l0 = quad_next(cur.l0.x), qh0_of_0 = quad_lane<0>(cur.h0.x);
      const uint32_t qh0_of_2 = quad_lane<2>(cur.h0.x);
      const uint32_t S0 = quad_lane<0>(cur.sd), S1 = quad_lane<1>(cur.sd);
      const uint32_t S2 = quad_lane<2>(cur.sd), S3 = quad_lane<3>(cur.sd);
      const uint32_t l8 = (2 * h + s) == 3 ? qh0_of_0 : next_l0;
      const uint32_t h8 = h ? S0 : qh0_of_2;
      const uint32_t lw[9] = {cur.l0.x, cur.l0.y, cur.l0.z, cur.l0.w, cur.l1.x, cur.l1.y, cur.l1.z, cur.l1.w, l8};
      const uint32_t hw[9] = {cur.h0.x, cur.h0.y, cur.h0.z, cur.h0.w, cur.h1.x, cur.h1.y, cur.h1.z, cur.h1.w, h8};
      // per sub-block (quarter s: l < 16, l >= 16; quarter s + 2: same) the
      // three plane sums of u X
      uint32_t a0[4] = {0u, 0u, 0u, 0u}, a1[4] = {0u, 0u, 0u, 0u};
      int a2[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t qlw = __builtin_amdgcn_alignbyte(lw[j + 1], lw[j], sh);
        const uint32_t qhw = __builtin_amdgcn_alignbyte(hw[j + 1], hw[j], sh) >> qh_shift;
        const uint32_t ulo = (qlw & 0x0F0F0F0Fu) | ((qhw & 0x03030303u) << 4);
        const uint32_t uhi = ((qlw >> 4) & 0x0F0F0F0Fu) | (((qhw >> 4) & 0x03030303u) << 4);
        const int ql_sub = j >> 2, qh_sub = 2 + (j >> 2);
        a0[ql_sub] = __builtin_amdgcn_udot4(ulo, xp.p0[j], a0[ql_sub], false);
        a1[ql_sub] = __builtin_amdgcn_udot4(ulo, xp.p1[j], a1[ql_sub], false);
        a2[ql_sub] = __builtin_amdgcn_sdot4(static_cast<int>(ulo), static_cast<int>(xp.p2[j]), a2[ql_sub], false);
        a0[qh_sub] = __builtin_amdgcn_udot4(uhi, xp.p0[8 + j], a0[qh_sub], false);
        a1[qh_sub] = __builtin_amdgcn_udot4(uhi, xp.p1[8 + j], a1[qh_sub], false);
        a2[qh_sub] = __builtin_amdgcn_sdot4(static_cast<int>(uhi), static_cast<int>(xp.p2[8 + j]), a2[qh_sub], false);
      }
      // sum u X = a0 + 2^8 a1 + 2^16 a2 (a0, a1 < 2^18, |a2| < 2^17)
      float P[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        P[q] = fmaf(65536.f, static_cast<float>(a2[q]),
                    fmaf(256.f, static_cast<float>(a1[q]), static_cast<float>(a0[q])));
      // scales 8h .. 8h+7 of the block; the lane's are 2s, 2s+1 (quarter s)
      // and 2s+4, 2s+5 (quarter s + 2)
      const uint32_t sc0 = __builtin_amdgcn_alignbyte(h ? S3 : S1, h ? S2 : S0, sh);
      const uint32_t sc1 = __builtin_amdgcn_alignbyte(h ? cur.tail4 : S2, h ? S3 : S1, sh);
      const uint32_t dbits = sh ? cur.tail4 >> 16 : cur.tail2;
      const float fl0 = scale_at(sc0, 2 * s), fl1 = scale_at(sc0, 2 * s + 1);
      const float fh0 = scale_at(sc1, 2 * s), fh1 = scale_at(sc1, 2 * s + 1);
      float v = fl0 * (P[0] - sx0);
      v = fmaf(fl1, P[1] - sx1, v);
      v = fmaf(fh0, P[2] - sx2, v);
      v = fmaf(fh1, P[3] - sx3, v);
      v *= half_bits_to_float(dbits) * xp.unit;
      // this register set is free: the row PF ahead goes in flight
      load_q6(rw, row_off(it + kQ6PF), h, s, raw[p]);
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
  // about one workgroup per compute unit (256), each slot a whole number of
  // prefetch groups
  const int unit = g.rs * kQ6PF;
  long long want = (static_cast<long long>(n) + 255) / 256;
  if (want > kQ6MaxRowsPerGroup) want = kQ6MaxRowsPerGroup;
  g.rpg = static_cast<int>((want + unit - 1) / unit * unit);
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
