// Dequant-fused Q4_K GEMV on the vector ALUs for one token, gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k (k divisible by 256);
// "realizar -- ffn.rs", fused_ffn_swiglu_gpu: the gate and up projections of
// one input followed by silu(gate) * up, done here in one pass.
//
// Activation-stationary layout.  A row of the matrix is cut into 4*(k/256)
// slices of 64 weights (one quarter g of a 256-block: quant bytes 32g..32g+31,
// sub-blocks 2g and 2g+1).  Each lane owns one slice position for the whole
// kernel and keeps the 64 matching activations (per token) in registers; the
// wavefront walks its rows, and at every row each lane streams its slice (two
// 16-byte loads plus the block header) and adds
//   d*sc_{2g} * sum q x  +  d*sc_{2g+1} * sum q x  -  dmin*(m_{2g} X_{2g} + m_{2g+1} X_{2g+1})
// where X are the slice's activation sums (precomputed once).  Nibbles are
// widened by v_cvt_pk_f32_fp8 (a byte 0..15 read as OCP e4m3 is q * 2^-9; the
// 2^9 goes into the scale).  Consecutive lanes own consecutive quarters, so a
// wavefront's loads cover 16 consecutive blocks of a row.
//
// Latency: each lane loads its own activations first and the weight loads of
// the next PF rows right behind them, so the activations arrive before the
// weights (loads return in order); the row loop then consumes weights as they
// stream in while later rows are already in flight.  A row that fits one
// wavefront is reduced by a butterfly over its lane segment and stored
// directly (no LDS, no barrier); wider rows add their per-wavefront sums in
// LDS at the end.  The summation order is fixed (deterministic).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kThreadsMax = 512;

template <bool BF16>
__device__ __forceinline__ float4 load_x4(const void* x, size_t idx) {
  if constexpr (BF16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + idx);
    return make_float4(bf16_bits_to_float(raw.x & 0xFFFFu), bf16_bits_to_float(raw.x >> 16),
                       bf16_bits_to_float(raw.y & 0xFFFFu), bf16_bits_to_float(raw.y >> 16));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + idx);
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

__device__ __forceinline__ void load_slice(const uint8_t* __restrict__ blk, int g, Slice& s) {
  const uint4 h = *reinterpret_cast<const uint4*>(blk);
  s.h = h.x; s.s0 = h.y; s.s1 = h.z; s.s2 = h.w;
  s.q0 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * g);
  s.q1 = *reinterpret_cast<const uint4*>(blk + 32 + 32 * g);
}

// acc += the four quants of `bits` (one nibble per byte) . x[0..3], as q * 2^-9
__device__ __forceinline__ float dot4(uint32_t bits, const float* x, float acc) {
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bits), false);
  const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bits), true);
  acc = fmaf(a.x, x[0], acc);
  acc = fmaf(a.y, x[1], acc);
  acc = fmaf(b.x, x[2], acc);
  acc = fmaf(b.y, x[3], acc);
  return acc;
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
  const float d = half_bits_to_float(s.h & 0xFFFFu) * 512.0f;  // cvt gives q * 2^-9
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

template <int MT>
__device__ __forceinline__ void slice_dot(const Slice& s, const FieldSel& f,
                                          const float (&xv)[MT][64], const float (&xsum)[MT][2],
                                          float (&out)[MT]) {
  float sc0, sc1, mn0, mn1;
  slice_scales(s, f, sc0, sc1, mn0, mn1);
  const uint32_t w[8] = {s.q0.x, s.q0.y, s.q0.z, s.q0.w, s.q1.x, s.q1.y, s.q1.z, s.q1.w};
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo = dot4(w[i] & 0x0F0F0F0Fu, &xv[t][4 * i], lo);
      hi = dot4((w[i] >> 4) & 0x0F0F0F0Fu, &xv[t][32 + 4 * i], hi);
    }
    float r = sc0 * lo;
    r = fmaf(sc1, hi, r);
    r = fmaf(-mn0, xsum[t][0], r);
    r = fmaf(-mn1, xsum[t][1], r);
    out[t] = r;
  }
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

template <int MT, bool GU, bool BF16, int PF>
__global__ __launch_bounds__(kThreadsMax) void gemv_xs_kernel(GemvArgs a, Geo geo) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int K = a.k / kQK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int expert = 0, mt = a.m;
  int xrow[MT], yrow[MT];
  if (a.slot_expert != nullptr) {
    const int slot = blockIdx.y;
    expert = a.slot_expert[slot];
    if (expert < 0) return;  // uniform over the workgroup, before any barrier
    mt = min(a.slot_count[slot], MT);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      xrow[t] = t < mt ? a.slot_x[slot * kMaxTokens + t] : 0;
      yrow[t] = t < mt ? a.slot_y[slot * kMaxTokens + t] : 0;
    }
  } else {
    mt = min(mt, MT);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      xrow[t] = t < mt ? t : 0;
      yrow[t] = t;
    }
  }
  const uint8_t* wg = a.w + static_cast<size_t>(expert) * a.mat_bytes;
  const uint8_t* wu = GU ? a.w_up + static_cast<size_t>(expert) * a.mat_bytes : nullptr;

  // this lane's row slot and slice
  int rslot, slice;
  if (geo.wr == 1) {
    rslot = wave * geo.rpw + lane / geo.lpr;
    slice = lane % geo.lpr;
  } else {
    rslot = wave / geo.wr;
    slice = (wave % geo.wr) * 64 + lane;
  }
  const bool lane_ok = slice < 4 * K && rslot < geo.step;
  const int b = lane_ok ? slice >> 2 : 0;
  const int g = slice & 3;
  FieldSel fsel;
  fsel.sh = 8u * static_cast<uint32_t>((2 * g) & 3);
  fsel.upper = g >= 2;

  const int row0 = blockIdx.x * geo.rows;
  const int rows = min(geo.rows, a.n - row0);
  const int iters = (rows + geo.step - 1) / geo.step;

  // 1. this lane's 64 activations per token, loaded first (loads return in
  //    order, so they are ready before the weights behind them)
  float xv[MT][64];
  const int xo = b * kQK + 64 * g;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (lane_ok && t < mt) v = load_x4<BF16>(a.x, static_cast<size_t>(xrow[t]) * a.ldx + xo + 4 * i);
      xv[t][4 * i] = v.x; xv[t][4 * i + 1] = v.y; xv[t][4 * i + 2] = v.z; xv[t][4 * i + 3] = v.w;
    }

  // 2. weight loads of the first PF steps
  Slice sg[PF], su[GU ? PF : 1];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int r = p * geo.step + rslot;
    if (lane_ok && r < rows) {
      const size_t off = (static_cast<size_t>(row0 + r) * K + b) * kBlockBytes;
      load_slice(wg + off, g, sg[p]);
      if constexpr (GU) load_slice(wu + off, g, su[p]);
    }
  }

  float xsum[MT][2];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      s0 += xv[t][i];
      s1 += xv[t][32 + i];
    }
    xsum[t][0] = s0;
    xsum[t][1] = s1;
  }

  // 3. row loop: consume step p while steps p+1 .. p+PF-1 are in flight; a
  //    row's slice partials are added over its lane segment with DPP lane
  //    permutes (every lane takes part, inactive ones contribute 0)
  float* part = smem;  // [GU?2:1][MT][rows][wr] when a row spans wavefronts
  const int seg = geo.wr == 1 ? geo.lpr : 64;
  for (int it0 = 0; it0 < iters; it0 += PF) {
    float o[PF][MT], ou[PF][GU ? MT : 1];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int it = it0 + p;
      const int r = it * geo.step + rslot;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        o[p][t] = 0.f;
        if constexpr (GU) ou[p][t] = 0.f;
      }
      if (it < iters && lane_ok && r < rows) {
        slice_dot<MT>(sg[p], fsel, xv, xsum, o[p]);
        if constexpr (GU) slice_dot<MT>(su[p], fsel, xv, xsum, ou[p]);
        const int rn = (it + PF) * geo.step + rslot;
        if (rn < rows) {
          const size_t off = (static_cast<size_t>(row0 + rn) * K + b) * kBlockBytes;
          load_slice(wg + off, g, sg[p]);
          if constexpr (GU) load_slice(wu + off, g, su[p]);
        }
      }
    }
    // add each row's slice partials over its lane segment (independent
    // chains for the PF rows, so they interleave)
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        o[p][t] = segment_sum_rt(o[p][t], seg);
        if constexpr (GU) ou[p][t] = segment_sum_rt(ou[p][t], seg);
      }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int it = it0 + p;
      const int r = it * geo.step + rslot;
      // the segment's last lane holds the row sum (it may be a padding lane)
      if (it < iters && rslot < geo.step && r < rows && (lane % seg) == seg - 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mt) {
            if (geo.wr == 1) {
              float out = o[p][t];
              if constexpr (GU) out = silu_mul(o[p][t], ou[p][t]);
              a.y[static_cast<size_t>(yrow[t]) * a.ldy + row0 + r] = out;
            } else {
              part[(t * rows + r) * geo.wr + slice / 64] = o[p][t];
              if constexpr (GU) part[((MT + t) * rows + r) * geo.wr + slice / 64] = ou[p][t];
            }
          }
        }
      }
    }
  }
  if (geo.wr == 1) return;  // uniform: no wavefront of this workgroup waits below
  __syncthreads();
  // 4. rows that span wavefronts: add the per-wavefront sums in order
  const int nthr = geo.waves * 64;
  for (int i = tid; i < rows * mt; i += nthr) {
    const int t = i / rows;
    const int r = i - t * rows;
    float s = 0.f, su_ = 0.f;
    for (int w = 0; w < geo.wr; ++w) {
      s += part[(t * rows + r) * geo.wr + w];
      if constexpr (GU) su_ += part[((MT + t) * rows + r) * geo.wr + w];
    }
    float out = s;
    if constexpr (GU) out = silu_mul(s, su_);
    a.y[static_cast<size_t>(yrow[t]) * a.ldy + row0 + r] = out;
  }
}

Geo make_geo(int n, int k, int slots) {
  Geo g{};
  const int K = k / kQK;
  const int l = 4 * K;
  if (l <= 64) {
    g.lpr = 1;
    while (g.lpr < l) g.lpr <<= 1;
    g.wr = 1;
    g.rpw = 64 / g.lpr;
    g.waves = 4;
    g.step = g.waves * g.rpw;
  } else {
    g.lpr = l;
    g.wr = (l + 63) / 64;
    g.rpw = 1;
    g.waves = g.wr * ((4 + g.wr - 1) / g.wr);  // at least 4 wavefronts
    if (g.waves > 8) g.waves = g.wr;
    g.step = g.waves / g.wr;
  }
  // rows per workgroup: about 256 workgroups over all slots, whole steps
  int want = (n * slots + 255) / 256;
  if (want < g.step) want = g.step;
  g.rows = (want + g.step - 1) / g.step * g.step;
  return g;
}

template <int MT, bool GU, bool BF16>
hipError_t launch_xs(const GemvArgs& a, hipStream_t stream) {
  constexpr int PF = (GU || MT > 1) ? 4 : 8;
  const int slots = a.slot_expert ? a.slots : 1;
  const Geo geo = make_geo(a.n, a.k, slots);
  const size_t lds = geo.wr == 1 ? 0
                                 : static_cast<size_t>(GU ? 2 : 1) * MT * geo.rows * geo.wr * sizeof(float);
  const dim3 grid((a.n + geo.rows - 1) / geo.rows, slots);
  gemv_xs_kernel<MT, GU, BF16, PF><<<grid, dim3(geo.waves * 64), lds, stream>>>(a, geo);
  return hipGetLastError();
}

}  // namespace

// The activations of a lane's slice stay in registers (64 floats per token):
// one token, any k up to 32768 (at most 8 wavefronts per row).
bool gemv_valu_fits(int m, int k, int n, int slots) {
  (void)n;
  (void)slots;
  return m == 1 && k <= 32768;
}

hipError_t launch_gemv_valu(const GemvArgs& a, hipStream_t stream) {
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
  if (gu) return bf ? launch_xs<1, true, true>(a, stream) : launch_xs<1, true, false>(a, stream);
  return bf ? launch_xs<1, false, true>(a, stream) : launch_xs<1, false, false>(a, stream);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int slots = a.slot_expert ? a.slots : 1;
  if (a.m <= 2 && gemv_valu_fits(a.m, a.k, a.n, slots)) return launch_gemv_valu(a, stream);
  return launch_gemv_mfma(a, stream);
}

}  // namespace q4k
