// Q8_1-activation decode GEMV on the vector ALUs, gfx950.
//
// "realizar -- ffn.rs", fused_ffn_swiglu_gpu_true_dp4a: the activations are
// quantised to Q8_1 (32 int8 values and one scale per block), each sub-block
// product with the Q4_K quants is an integer dot product of packed bytes,
// and the scales are applied afterwards.  For token t, weight row j and the
// 32-value sub-block s:
//   P = sum_{i<32} q_w * q_a                   (v_dot4_i32_i8, exact in int32)
//   y[t][j] += (d*sc_s) * (d_a * P)  -  (dmin*m_s) * (d_a * S)
// with S the integer block sum stored next to d_a.  This is the product
// q4k_mmq computes, for the few tokens of a decode step, where a GEMM tile
// would leave most of the matrix cores idle and the weight stream is what
// costs.
//
// Activation-stationary layout.  A row is cut into 4*(k/256) slices of 64
// weights (quarter g of a 256-block: quant bytes 32g..32g+31, whose low
// nibbles are sub-block 2g and high nibbles sub-block 2g+1).  Each lane owns
// one slice position for the whole kernel and holds the 64 activation quants
// of that position for every token in registers (16 words per token), with
// d_a and d_a*S of its two sub-blocks.  A wavefront covers 16 consecutive
// blocks of a row; a row wider than that spans wr wavefronts, whose sums meet
// in LDS.  Per row a lane loads 48 bytes (the 16-byte block header and its 32
// quant bytes, raw buffer loads that read zeros past the last row); PF rows
// are in flight per wavefront.  Lane sums are reduced across the row's lanes
// in a fixed order (deterministic): lane swaps between half-waves and rows
// halve the number of token values per step, then DPP within rows.  Tokens are processed MT at a
// time (1, 2, 4 or 8); the missing ones read zeros and are not stored.
//
// Gate/up form (GU): the same pass over two matrices of one shape, row j of
// both at once, storing silu(gate_j) * up_j ("realizar -- ffn.rs", the
// DP4A FFN's gate and up GEMVs followed by its SwiGLU step).
#include "lane_reduce.hpp"
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kQ8Threads = 512;
constexpr int kQ8MaxRowsPerGroup = 64;

struct Q8Geo {
  int wr;    // wavefronts per row
  int rs;    // row slots per workgroup (rows in flight side by side)
  int rpg;   // rows per workgroup (a multiple of rs)
};

struct RowRaw {
  uint4 h;   // block header
  uint4 q0;  // quant bytes 32g .. 32g+15
  uint4 q1;  // quant bytes 32g+16 .. 32g+31
};

__device__ __forceinline__ void load_row(rsrc_t r, uint32_t off, int g, RowRaw& raw) {
  raw.h = buf_load16(r, off);
  const uint32_t q = off == kOob ? kOob : off + 16u + 32u * static_cast<uint32_t>(g);
  raw.q0 = buf_load16(r, q);
  raw.q1 = buf_load16(r, q == kOob ? kOob : q + 16u);
}


template <int MT, int PF, bool GU>
__global__ __launch_bounds__(kQ8Threads) void q8_gemv_kernel(const uint8_t* __restrict__ w,
                                                             const uint8_t* __restrict__ wu,
                                                             const int8_t* __restrict__ qs,
                                                             const uint32_t* __restrict__ ds,
                                                             float* __restrict__ y, int m, int n,
                                                             int k, Q8Geo geo) {
  constexpr int NM = GU ? 2 : 1;  // matrices per pass
  extern __shared__ __attribute__((aligned(16))) float part[];  // [rpg][wr][NM][MT]
  const int K = k >> 8;
  const int S = 4 * K;
  const int nsub = k >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / geo.wr;  // uniform
  const int wpart = wave - slot * geo.wr;
  const int slice = wpart * 64 + lane;
  const bool lane_ok = slice < S;
  const int b = lane_ok ? slice >> 2 : 0;
  const int g = slice & 3;

  // 1. this lane's activations: token t, k = 256b + 64g .. +63 (sub-blocks
  //    8b+2g and 8b+2g+1), read once
  const rsrc_t rq = make_rsrc(qs, static_cast<uint32_t>(m) * static_cast<uint32_t>(k));
  const rsrc_t rd = make_rsrc(ds, static_cast<uint32_t>(m) * static_cast<uint32_t>(nsub) * 4u);
  uint32_t xa[MT][16];
  float da0[MT], da1[MT], sa0[MT], sa1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const uint32_t base = lane_ok ? static_cast<uint32_t>(t) * k + 256u * b + 64u * g : kOob;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = buf_load16(rq, base == kOob ? kOob : base + 16u * c);
      xa[t][4 * c] = v.x;
      xa[t][4 * c + 1] = v.y;
      xa[t][4 * c + 2] = v.z;
      xa[t][4 * c + 3] = v.w;
    }
    const uint32_t dofs = lane_ok ? (static_cast<uint32_t>(t) * nsub + 8u * b + 2u * g) * 4u : kOob;
    const uint2 dw = buf_load8(rd, dofs);
    da0[t] = half_bits_to_float(dw.x & 0xFFFFu);
    da1[t] = half_bits_to_float(dw.y & 0xFFFFu);
    sa0[t] = da0[t] * static_cast<float>(static_cast<int16_t>(dw.x >> 16));  // exact
    sa1[t] = da1[t] * static_cast<float>(static_cast<int16_t>(dw.y >> 16));
  }

  // 2. the workgroup's rows: slot `slot` takes rows slot, slot + rs, ...
  const int row0 = blockIdx.x * geo.rpg;
  const int rows = min(geo.rpg, n - row0);
  const size_t wofs = static_cast<size_t>(row0) * K * kBlockBytes;
  const uint32_t span = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  const rsrc_t rw = make_rsrc(w + wofs, span);
  const rsrc_t rwu = make_rsrc(GU ? wu + wofs : w, GU ? span : 0u);
  const uint32_t stride = static_cast<uint32_t>(geo.rs) * static_cast<uint32_t>(K) * kBlockBytes;
  const uint32_t base = static_cast<uint32_t>(slot * K + b) * kBlockBytes;
  const int nit = (rows - slot + geo.rs - 1) / geo.rs;  // rows of this slot (uniform)
  auto row_off = [&](int it) -> uint32_t {
    return lane_ok && it < nit ? base + static_cast<uint32_t>(it) * stride : kOob;
  };
  const int wgroups = (nit + PF - 1) / PF;

  RowRaw raw[PF], rawu[GU ? PF : 1];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_row(rw, row_off(p), g, raw[p]);
    if constexpr (GU) load_row(rwu, row_off(p), g, rawu[p]);
  }
  int hold_tok;
  bool holder;
  token_map<MT>(lane, hold_tok, holder);

  // this lane's share of one row for every token: the two sub-block products
  // scaled in f32
  auto row_dot = [&](const RowRaw& rr, float (&acc)[MT]) {
    const uint4 h = rr.h;
    const float d = half_bits_to_float(h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(h.x >> 16);
    uint32_t sc0, mn0, sc1, mn1;
    scale_min_rt(h, 2 * g, sc0, mn0);
    scale_min_rt(h, 2 * g + 1, sc1, mn1);
    const float ws0 = d * static_cast<float>(sc0), ws1 = d * static_cast<float>(sc1);  // exact
    const float wm0 = dmin * static_cast<float>(mn0), wm1 = dmin * static_cast<float>(mn1);
    const uint32_t qw[8] = {rr.q0.x, rr.q0.y, rr.q0.z, rr.q0.w, rr.q1.x, rr.q1.y, rr.q1.z, rr.q1.w};
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = qw[i] & 0x0F0F0F0Fu;         // sub-block 2g, positions 4i .. 4i+3
      hi[i] = (qw[i] >> 4) & 0x0F0F0F0Fu;  // sub-block 2g+1, same positions
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      int p0 = 0, p1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p0 = __builtin_amdgcn_sdot4(static_cast<int>(lo[i]), static_cast<int>(xa[t][i]), p0, false);
        p1 = __builtin_amdgcn_sdot4(static_cast<int>(hi[i]), static_cast<int>(xa[t][8 + i]), p1, false);
      }
      float v = ws0 * (da0[t] * static_cast<float>(p0));
      v = fmaf(ws1, da1[t] * static_cast<float>(p1), v);
      v = fmaf(-wm0, sa0[t], v);
      v = fmaf(-wm1, sa1[t], v);
      acc[t] = lane_ok ? v : 0.f;
    }
  };

  for (int grp = 0; grp < wgroups; ++grp) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int it = grp * PF + p;
      // the next row of each register set is in flight while this one is used
      float acc[MT], accu[MT];
      const RowRaw cur = raw[p];
      load_row(rw, row_off(it + PF), g, raw[p]);
      row_dot(cur, acc);
      if constexpr (GU) {
        const RowRaw curu = rawu[p];
        load_row(rwu, row_off(it + PF), g, rawu[p]);
        row_dot(curu, accu);
      }
      // row sums over the wavefront's lanes (one lane per token holds a
      // total), then over the row's wavefronts
      const float tot = row_reduce<MT>(acc, lane);
      float totu = 0.f;
      if constexpr (GU) totu = row_reduce<MT>(accu, lane);
      if (it < nit && holder) {
        const int r = slot + it * geo.rs;
        if (geo.wr == 1) {
          if (hold_tok < m) y[static_cast<size_t>(hold_tok) * n + row0 + r] = GU ? silu_mul(tot, totu) : tot;
        } else {
          part[((r * geo.wr + wpart) * NM) * MT + hold_tok] = tot;
          if constexpr (GU) part[((r * geo.wr + wpart) * NM + 1) * MT + hold_tok] = totu;
        }
      }
    }
  }
  if (geo.wr > 1) {
    __syncthreads();
    for (int e = tid; e < rows * MT; e += blockDim.x) {
      const int r = e / MT, t = e - r * MT;
      float s = 0.f, su = 0.f;
      for (int q = 0; q < geo.wr; ++q) {
        s += part[((r * geo.wr + q) * NM) * MT + t];
        if constexpr (GU) su += part[((r * geo.wr + q) * NM + 1) * MT + t];
      }
      if (t < m) y[static_cast<size_t>(t) * n + row0 + r] = GU ? silu_mul(s, su) : s;
    }
  }
}

Q8Geo make_q8_geo(int n, int k) {
  Q8Geo g{};
  const int S = 4 * (k / kQK);
  g.wr = (S + 63) / 64;
  g.rs = g.wr >= 4 ? 1 : (4 + g.wr - 1) / g.wr;
  // about 256 workgroups (one per CU), at most 64 rows each, whole slots
  long long want = (static_cast<long long>(n) + 255) / 256;
  if (want < g.rs) want = g.rs;
  if (want > kQ8MaxRowsPerGroup) want = kQ8MaxRowsPerGroup;
  g.rpg = static_cast<int>((want + g.rs - 1) / g.rs * g.rs);
  return g;
}

// rows in flight per wavefront and matrix: 4, or 2 at 8 tokens; the gate/up
// form keeps half as many of each matrix
template <int MT, bool GU>
hipError_t launch_mt(const uint8_t* w, const uint8_t* wu, const int8_t* qs, const uint32_t* ds, float* y,
                     int m, int n, int k, hipStream_t stream) {
  constexpr int PF = GU && MT == 1 ? 4 : (MT >= 8 ? 2 : 4) / (GU ? 2 : 1);
  constexpr int NM = GU ? 2 : 1;
  const Q8Geo g = make_q8_geo(n, k);
  const size_t lds = g.wr > 1 ? static_cast<size_t>(g.rpg) * g.wr * NM * MT * sizeof(float) : 0;
  const dim3 grid((n + g.rpg - 1) / g.rpg);
  q8_gemv_kernel<MT, PF, GU><<<grid, dim3(64 * g.wr * g.rs), lds, stream>>>(w, wu, qs, ds, y, m, n, k, g);
  return hipGetLastError();
}

template <bool GU>
hipError_t launch_tokens(const uint8_t* w, const uint8_t* wu, const int8_t* qs, const uint32_t* ds,
                         float* y, int m, int n, int k, hipStream_t stream) {
  if (m < 1 || m > kMaxTokens || k < kQK || k % kQK || k > 32768 || n < 1) return hipErrorInvalidValue;
  if (m == 1) return launch_mt<1, GU>(w, wu, qs, ds, y, m, n, k, stream);
  if (m == 2) return launch_mt<2, GU>(w, wu, qs, ds, y, m, n, k, stream);
  if (m <= 4) return launch_mt<4, GU>(w, wu, qs, ds, y, m, n, k, stream);
  return launch_mt<8, GU>(w, wu, qs, ds, y, m, n, k, stream);
}

}  // namespace

hipError_t launch_q8_gemv(const uint8_t* w, const int8_t* qs, const uint32_t* ds, float* y, int m,
                          int n, int k, hipStream_t stream) {
  return launch_tokens<false>(w, nullptr, qs, ds, y, m, n, k, stream);
}

hipError_t launch_q8_gemv_gu(const uint8_t* w_gate, const uint8_t* w_up, const int8_t* qs,
                             const uint32_t* ds, float* h, int m, int n, int k, hipStream_t stream) {
  return launch_tokens<true>(w_gate, w_up, qs, ds, h, m, n, k, stream);
}

}  // namespace q4k
