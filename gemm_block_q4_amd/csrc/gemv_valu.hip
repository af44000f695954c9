// Dequant-fused Q4_K GEMV on the vector ALUs for one token, gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k (k divisible by 256);
// "realizar -- ffn.rs", fused_ffn_swiglu_gpu: the gate and up projections of
// one input followed by silu(gate) * up, done here in one pass.
//
// Activation-stationary layout.  A row of the matrix is cut into 4*(k/256)
// slices of 64 weights (one quarter g of a 256-block: quant bytes 32g..32g+31,
// low nibbles = sub-block 2g, high nibbles = sub-block 2g+1).  Each lane owns
// one slice position for the whole kernel; the wavefront walks its rows and at
// every row each lane streams its slice (two 16-byte loads plus the block
// header) and adds
//   d*sc_{2g} * sum q x  +  d*sc_{2g+1} * sum q x  -  dmin*(m_{2g} X_{2g} + m_{2g+1} X_{2g+1})
// where X are the f32 sums of the slice's two halves of x.  Consecutive lanes
// own consecutive quarters, so a wavefront's loads cover 16 consecutive blocks
// of a row.
//
// Integer inner products.  The activations are fixed for the whole kernel, so
// the workgroup converts them once: each 64-value slice gets a power-of-two
// scale 2^e with every |x| < 2^e, and each value becomes the integer
// a = rint(x * 2^(21-e)), |a| <= 2^21 (21 significant bits relative to the
// slice maximum).  One FMA with the constant 1.5 * 2^23 leaves a + 2^22 in the
// low 23 bits of the f32 result; its three bytes u0, u1, u2 give
// a = u0 + 2^8 u1 + 2^16 (u2 - 64), stored as two unsigned byte planes and one
// signed plane (u2 - 64 lies in [-32, 32]).  A masked nibble word is four
// bytes below 16, so four weights times one plane are one v_dot4 (unsigned
// for planes 0, 1, signed for plane 2), and the three plane sums of a
// sub-block combine exactly in int32 as S0 + 2^8 S1 + 2^16 S2, scaled by
// 2^(e-21).  No weight is ever converted to floating point.
//
// Latency: each thread loads its share of the activations first and the
// weight loads of the next PF rows right behind them (loads return in order);
// the workgroup writes the digits to LDS (one barrier), every lane copies its
// slice's 48 digit words to registers, and the row loop then consumes weights
// as they stream in.  A row that fits one wavefront is reduced with DPP lane
// permutes and stored directly; wider rows add their per-wavefront sums in LDS
// at the end.  The summation order is fixed (deterministic).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kThreadsMax = 512;
constexpr int kWavesNarrow = 4;  // wavefronts per workgroup when a row fits one wavefront
constexpr int kWavesWide = 8;    // at most this many when a row spans wavefronts
constexpr int kUnitsEarly = 2;  // 16-value activation units per thread loaded before the weights
constexpr size_t kLdsMax = 160 * 1024;

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

// The quarter of one block a lane streams per row.
struct Slice {
  uint32_t h;   // d | dmin << 16
  uint32_t s0;  // scales[0..3]
  uint32_t s1;  // scales[4..7]
  uint32_t s2;  // scales[8..11]
  uint4 q0, q1; // quant bytes 32g .. 32g+31
};

// Slice g of the block at byte offset `off` of the resource (kOob: zeros).
__device__ __forceinline__ void load_slice(rsrc_t r, uint32_t off, int g, Slice& s) {
  const uint4 h = buf_load16(r, off);
  s.h = h.x; s.s0 = h.y; s.s1 = h.z; s.s2 = h.w;
  const uint32_t q = off + 32u * static_cast<uint32_t>(g);
  s.q0 = buf_load16(r, q + 16u);
  s.q1 = buf_load16(r, q + 32u);
}

// Lane permutes on the VALU (no LDS round trip).  Lanes whose source is out of
// range read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, true));
}

// Sum over aligned segments of SEG lanes (SEG a power of two <= 64); the
// total lands in the last lane of each segment.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v) {
  if constexpr (SEG >= 2) v += dpp<0xB1>(v);        // quad_perm(1,0,3,2)
  if constexpr (SEG >= 4) v += dpp<0x4E>(v);        // quad_perm(2,3,0,1)
  if constexpr (SEG >= 8) v += dpp<0x114>(v);       // row_shr:4
  if constexpr (SEG >= 16) v += dpp<0x118>(v);      // row_shr:8
  if constexpr (SEG >= 32) v += dpp<0x142, 0xA>(v); // row_bcast:15 into rows 1, 3
  if constexpr (SEG >= 64) v += dpp<0x143, 0xC>(v); // row_bcast:31 into rows 2, 3
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

// Per-lane constants of the 6-bit field extraction for sub-blocks 2g, 2g+1:
// byte u = (2g) & 3 of the scale words, and whether the pair is in the upper
// half (sub-blocks 4..7).
struct FieldSel {
  uint32_t sh;   // 8 * u
  bool upper;
};

__device__ __forceinline__ void slice_scales(const Slice& s, const FieldSel& f, float& sc0,
                                             float& sc1, float& mn0, float& mn1) {
  const float d = half_bits_to_float(s.h & 0xFFFFu);
  const float dmin = half_bits_to_float(s.h >> 16);
  const uint32_t a = s.s0 >> f.sh, b = s.s1 >> f.sh, c = s.s2 >> f.sh;
  uint32_t c0, c1, m0, m1;
  if (f.upper) {
    // scale = low nibble of scales[8+u] | top bits of scales[u]; min = high
    // nibble of scales[8+u] | top bits of scales[4+u]
    c0 = (c & 15u) | ((a >> 6) & 3u) << 4;
    c1 = ((c >> 8) & 15u) | ((a >> 14) & 3u) << 4;
    m0 = ((c >> 4) & 15u) | ((b >> 6) & 3u) << 4;
    m1 = ((c >> 12) & 15u) | ((b >> 14) & 3u) << 4;
  } else {
    c0 = a & 63u;
    c1 = (a >> 8) & 63u;
    m0 = b & 63u;
    m1 = (b >> 8) & 63u;
  }
  sc0 = d * static_cast<float>(c0);
  sc1 = d * static_cast<float>(c1);
  mn0 = dmin * static_cast<float>(m0);
  mn1 = dmin * static_cast<float>(m1);
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

__device__ __forceinline__ float slice_dot(const Slice& s, const FieldSel& f, const XSlice& x) {
  float sc0, sc1, mn0, mn1;
  slice_scales(s, f, sc0, sc1, mn0, mn1);
  const uint32_t w[8] = {s.q0.x, s.q0.y, s.q0.z, s.q0.w, s.q1.x, s.q1.y, s.q1.z, s.q1.w};
  const float lo = static_cast<float>(plane_dot(w, 0, x, 0));  // sub-block 2g: low nibbles
  const float hi = static_cast<float>(plane_dot(w, 4, x, 8));  // sub-block 2g+1: high nibbles
  float r = fmaf(sc1, hi, sc0 * lo) * x.scale;
  r = fmaf(-mn0, x.sum0, r);
  r = fmaf(-mn1, x.sum1, r);
  return r;
}

// Launch geometry (all per workgroup):
//   lanes per row  lpr = 4 * (k/256) slices, rounded up to a power of two when
//   a row fits one wavefront (so rows are aligned lane segments);
//   wr   = wavefronts per row (1 when lpr <= 64);
//   rpw  = rows per wavefront per step (64 / lpr when wr == 1, else 1);
//   step = rows per workgroup per step; rows = rows per workgroup.
struct Geo {
  int lpr, wr, rpw, waves, step, rows;
};

// LDS words: digit planes [S][48] and slice info [S][4] (scale, sum0, sum1,
// unused), then the row partials when a row spans wavefronts.
__host__ __device__ __forceinline__ size_t x_words(int slices) { return static_cast<size_t>(slices) * 52; }

// Converts one 16-value activation unit u (values 16u .. 16u+15, quarter u & 3
// of slice u >> 2) to byte planes in LDS.  The four units of a slice are an
// aligned lane quad, so the slice maximum and the half sums are quad DPP
// reductions; every lane of the quad must execute this (uniform control flow).
__device__ __forceinline__ void convert_unit(const float4 (&xr)[4], int u, bool valid,
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
  amax = fmaxf(amax, dpp<0xB1>(amax));
  amax = fmaxf(amax, dpp<0x4E>(amax));
  sum += dpp<0xB1>(sum);  // units 0+1 and 2+3: the two 32-value halves
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
  uint32_t* base = dig + static_cast<size_t>(s) * 48 + 4 * qq;
  *reinterpret_cast<uint4*>(base) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
  *reinterpret_cast<uint4*>(base + 16) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
  *reinterpret_cast<uint4*>(base + 32) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
  if (qq == 0) {
    // amax - amax is 0 for a finite maximum and NaN otherwise
    xinfo[4 * s] = __uint_as_float(static_cast<uint32_t>(127 - 21 + e) << 23) + (amax - amax);
    xinfo[4 * s + 1] = sum;
  } else if (qq == 2) {
    xinfo[4 * s + 2] = sum;
  }
}

template <bool GU, bool BF16, int PF, bool SEG64>
__global__ __launch_bounds__(kThreadsMax) void gemv_d4_kernel(GemvArgs a, Geo geo) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem_u[];
  const int K = a.k / kQK;
  const int S = 4 * K;  // slices per row
  const int units = 4 * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthr = geo.waves * 64;

  int expert = 0, xrow = 0, yrow = 0;
  if (a.slot_expert != nullptr) {
    const int slot = blockIdx.y;
    expert = a.slot_expert[slot];
    // uniform over the workgroup, before any barrier
    if (expert < 0 || a.slot_count[slot] < 1) return;
    xrow = a.slot_x[slot * kMaxTokens];
    yrow = a.slot_y[slot * kMaxTokens];
  }

  // this lane's row slot and slice
  int rslot, slice;
  if (geo.wr == 1) {
    rslot = wave * geo.rpw + lane / geo.lpr;
    slice = lane % geo.lpr;
  } else {
    rslot = wave / geo.wr;
    slice = (wave % geo.wr) * 64 + lane;
  }
  const bool lane_ok = slice < S && rslot < geo.step;
  const int b = lane_ok ? slice >> 2 : 0;
  const int g = slice & 3;
  FieldSel fsel;
  fsel.sh = 8u * static_cast<uint32_t>((2 * g) & 3);
  fsel.upper = g >= 2;

  const int row0 = blockIdx.x * geo.rows;
  const int rows = min(geo.rows, a.n - row0);
  const int iters = (rows + geo.step - 1) / geo.step;

  // buffer resources: this workgroup's rows of the matrices (under 2^31 bytes
  // by construction of the geometry) and the token's activation row
  const size_t wofs = static_cast<size_t>(expert) * a.mat_bytes +
                      static_cast<size_t>(row0) * K * kBlockBytes;
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  const rsrc_t rg = make_rsrc(a.w + wofs, wbytes);
  const rsrc_t ru = GU ? make_rsrc(a.w_up + wofs, wbytes) : rg;
  const size_t xel = static_cast<size_t>(xrow) * a.ldx;
  const rsrc_t rx = BF16 ? make_rsrc(static_cast<const uint16_t*>(a.x) + xel, 2u * a.k)
                         : make_rsrc(static_cast<const float*>(a.x) + xel, 4u * a.k);
  // byte offset of this lane's block in row r of the workgroup, kOob past the end
  auto row_off = [&](int r) -> uint32_t {
    return lane_ok && r < rows ? static_cast<uint32_t>(r * K + b) * kBlockBytes : kOob;
  };
  auto unit_off = [&](int u, int c) -> uint32_t {
    return u < units ? static_cast<uint32_t>(16 * u + 4 * c) : kOob;
  };

  // 1. the first activation units of this thread, loaded before any weight
  float4 xr[kUnitsEarly][4];
#pragma unroll
  for (int j = 0; j < kUnitsEarly; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) xr[j][c] = load_x4<BF16>(rx, unit_off(tid + j * nthr, c));

  // 2. weight loads of the first PF steps
  Slice sg[PF], su[GU ? PF : 1];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const uint32_t off = row_off(p * geo.step + rslot);
    load_slice(rg, off, g, sg[p]);
    if constexpr (GU) load_slice(ru, off, g, su[p]);
  }

  // 3. activations -> digits in LDS, once per workgroup (the loop bounds are
  //    uniform, so every quad converts together)
  uint32_t* dig = smem_u;                                                         // [S][48]
  float* xinfo = reinterpret_cast<float*>(smem_u + static_cast<size_t>(S) * 48);  // [S][4]
#pragma unroll
  for (int j = 0; j < kUnitsEarly; ++j) {
    if (j * nthr >= units) break;
    const int u = tid + j * nthr;
    convert_unit(xr[j], u, u < units, dig, xinfo);
  }
  for (int j = kUnitsEarly; j * nthr < units; ++j) {
    const int u = tid + j * nthr;
    float4 xl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) xl[c] = load_x4<BF16>(rx, unit_off(u, c));
    convert_unit(xl, u, u < units, dig, xinfo);
  }
  __syncthreads();
  XSlice xs;
  {
    const uint32_t* base = dig + static_cast<size_t>(lane_ok ? slice : 0) * 48;
#pragma unroll
    for (int d = 0; d < 3; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(base + 16 * d + 4 * i);
        xs.dg[d][4 * i] = t4.x; xs.dg[d][4 * i + 1] = t4.y;
        xs.dg[d][4 * i + 2] = t4.z; xs.dg[d][4 * i + 3] = t4.w;
      }
    const float4 inf = *reinterpret_cast<const float4*>(xinfo + 4 * (lane_ok ? slice : 0));
    xs.scale = inf.x; xs.sum0 = inf.y; xs.sum1 = inf.z;
  }

  // 4. row loop: consume step p while steps p+1 .. p+PF-1 are in flight.  The
  //    loads are never under a branch (rows past the end read kOob); inactive
  //    lanes contribute 0 to the DPP segment sums.
  float* part = reinterpret_cast<float*>(smem_u + x_words(S));  // [GU?2:1][rows][wr]
  const int seg = SEG64 ? 64 : (geo.wr == 1 ? geo.lpr : 64);
  auto finish = [&](float (&o)[PF], float (&ou)[PF], int it0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      o[p] = SEG64 ? segment_sum<64>(o[p]) : segment_sum_rt(o[p], seg);
      if constexpr (GU) ou[p] = SEG64 ? segment_sum<64>(ou[p]) : segment_sum_rt(ou[p], seg);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int it = it0 + p;
      const int r = it * geo.step + rslot;
      // the segment's last lane holds the row sum (it may be a padding lane)
      if (it < iters && rslot < geo.step && r < rows && (lane % seg) == seg - 1) {
        if (geo.wr == 1) {
          float out = o[p];
          if constexpr (GU) out = silu_mul(o[p], ou[p]);
          a.y[static_cast<size_t>(yrow) * a.ldy + row0 + r] = out;
        } else {
          part[r * geo.wr + slice / 64] = o[p];
          if constexpr (GU) part[(rows + r) * geo.wr + slice / 64] = ou[p];
        }
      }
    }
  };
  int it0 = 0;
  for (; it0 + PF <= iters; it0 += PF) {
    float o[PF], ou[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int r = (it0 + p) * geo.step + rslot;
      const bool ok = lane_ok && r < rows;
      const float v = slice_dot(sg[p], fsel, xs);
      o[p] = ok ? v : 0.f;
      ou[p] = 0.f;
      if constexpr (GU) {
        const float vu = slice_dot(su[p], fsel, xs);
        ou[p] = ok ? vu : 0.f;
      }
      const uint32_t off = row_off((it0 + p + PF) * geo.step + rslot);
      load_slice(rg, off, g, sg[p]);
      if constexpr (GU) load_slice(ru, off, g, su[p]);
    }
    finish(o, ou, it0);
  }
  if (it0 < iters) {  // the last, partial group: nothing left to prefetch
    float o[PF], ou[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      o[p] = 0.f;
      ou[p] = 0.f;
      if (it0 + p < iters) {  // uniform
        const int r = (it0 + p) * geo.step + rslot;
        const bool ok = lane_ok && r < rows;
        const float v = slice_dot(sg[p], fsel, xs);
        o[p] = ok ? v : 0.f;
        if constexpr (GU) {
          const float vu = slice_dot(su[p], fsel, xs);
          ou[p] = ok ? vu : 0.f;
        }
      }
    }
    finish(o, ou, it0);
  }
  if (geo.wr == 1) return;  // uniform: no wavefront of this workgroup waits below
  __syncthreads();
  // 5. rows that span wavefronts: add the per-wavefront sums in order
  for (int r = tid; r < rows; r += nthr) {
    float s = 0.f, su_ = 0.f;
    for (int w = 0; w < geo.wr; ++w) {
      s += part[r * geo.wr + w];
      if constexpr (GU) su_ += part[(rows + r) * geo.wr + w];
    }
    float out = s;
    if constexpr (GU) out = silu_mul(s, su_);
    a.y[static_cast<size_t>(yrow) * a.ldy + row0 + r] = out;
  }
}

size_t lds_bytes(const Geo& geo, int k, bool gu) {
  size_t words = x_words(4 * (k / kQK));
  if (geo.wr > 1) words += static_cast<size_t>(gu ? 2 : 1) * geo.rows * geo.wr;
  return words * sizeof(uint32_t);
}

Geo make_geo(int n, int k, int slots, bool gu) {
  Geo g{};
  const int K = k / kQK;
  const int l = 4 * K;
  if (l <= 64) {
    g.lpr = 1;
    while (g.lpr < l) g.lpr <<= 1;
    g.wr = 1;
    g.rpw = 64 / g.lpr;
    g.waves = kWavesNarrow;
    g.step = g.waves * g.rpw;
  } else {
    g.lpr = l;
    g.wr = (l + 63) / 64;
    g.rpw = 1;
    g.waves = g.wr * (g.wr >= kWavesWide ? 1 : kWavesWide / g.wr);  // whole rows
    g.step = g.waves / g.wr;
  }
  // rows per workgroup: about 256 workgroups over all slots, whole steps,
  // and no more row partials than fit next to the digits in LDS
  long long want = (static_cast<long long>(n) * slots + 255) / 256;
  if (want > n) want = n;
  if (want < g.step) want = g.step;
  g.rows = static_cast<int>((want + g.step - 1) / g.step * g.step);
  const int cap_bytes = static_cast<int>((static_cast<size_t>(kOob) - 1) / (static_cast<size_t>(K) * kBlockBytes)) /
                        g.step * g.step;
  if (g.rows > cap_bytes) g.rows = cap_bytes;
  if (g.wr > 1) {
    const size_t free_words = kLdsMax / sizeof(uint32_t) - x_words(l);
    const int cap = static_cast<int>(free_words / (static_cast<size_t>(gu ? 2 : 1) * g.wr)) / g.step * g.step;
    if (g.rows > cap) g.rows = cap;
  }
  return g;
}

template <bool GU, bool BF16>
hipError_t launch_d4(const GemvArgs& a, hipStream_t stream) {
  constexpr int PF = GU ? 2 : 4;
  const int slots = a.slot_expert ? a.slots : 1;
  const Geo geo = make_geo(a.n, a.k, slots, GU);
  const size_t lds = lds_bytes(geo, a.k, GU);
  if (geo.rows < geo.step || lds > kLdsMax) return hipErrorInvalidValue;
  // rows of exactly one wavefront reduce over all 64 lanes
  const bool seg64 = geo.wr > 1 || geo.lpr == 64;
  auto kern = seg64 ? gemv_d4_kernel<GU, BF16, PF, true> : gemv_d4_kernel<GU, BF16, PF, false>;
  static bool big_lds = false;  // the opt-in is per kernel and stays set
  if (lds > 64 * 1024 && !big_lds) {
    for (auto kv : {gemv_d4_kernel<GU, BF16, PF, true>, gemv_d4_kernel<GU, BF16, PF, false>}) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kv),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(kLdsMax));
      if (e != hipSuccess) return e;
    }
    big_lds = true;
  }
  const dim3 grid((a.n + geo.rows - 1) / geo.rows, slots);
  kern<<<grid, dim3(geo.waves * 64), lds, stream>>>(a, geo);
  return hipGetLastError();
}

}  // namespace

// One token and k up to 32768: at most 8 wavefronts per row, and the digits of
// all activations (208 bytes per 64 values, 104 KiB at k = 32768) fit in LDS.
bool gemv_valu_fits(int m, int k) { return m == 1 && k <= 32768; }

hipError_t launch_gemv_valu(const GemvArgs& a, hipStream_t stream) {
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
  if (gu) return bf ? launch_d4<true, true>(a, stream) : launch_d4<true, false>(a, stream);
  return bf ? launch_d4<false, true>(a, stream) : launch_d4<false, false>(a, stream);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  if (gemv_valu_fits(a.m, a.k)) return launch_gemv_valu(a, stream);
  return launch_gemv_mfma(a, stream);
}

}  // namespace q4k
