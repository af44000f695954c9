// Dequant-fused Q4_K GEMV on the matrix cores (3..8 tokens), gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k; "realizar -- ffn.rs",
// fused_ffn_swiglu_gpu: gate and up GEMVs, silu(gate) * up, then the down
// GEMV.  Here the gate and up GEMVs run in one pass over both matrices and
// the silu * mul is applied before the single store.
//
// The dot products run on the matrix cores (v_mfma_f32_16x16x32_f16) with
// exact operands:
//  * weights: for sub-block j the product sc_j * q is an integer <= 945,
//    exact in binary16, so each 256-block is one chain of 8 K=32 steps whose
//    f32 sum is multiplied by d once; the min term sum_j m_j * X_j (X_j the
//    activation sum of sub-block j, carried as X_j * 2^-6 against m_j * 2^6
//    so that it fits binary16) is one more K=32 step whose result is
//    multiplied by dmin;
//  * activations: per token and 256-block, x is scaled by 2^sh (sh chosen so
//    the block maximum lands in [2^14, 2^15)) and split into two binary16
//    halves hi + lo that carry 22 significant bits; both halves go through
//    the same weight operand, and the block result is scaled back by 2^-sh.
// The relative error of a row result is thus a few 2^-22 of ||w|| ||x||.
//
// Work decomposition: a workgroup (4 wavefronts) owns 16 output rows; the
// k/256 blocks are split into four contiguous ranges, one per wavefront.
// Lane l holds weight row n0 + l%16 and the 64 weights 64*(l/16) .. +63 of
// each block (32 contiguous quant bytes, two 16-byte loads), i.e. the K
// index 8*(l/16)+i of step s is weight 64*(l/16) + 8*s + i; the activation
// operand uses the same K mapping with the token in place of the row.  Each
// wavefront converts its own activation range, four blocks at a time, into
// LDS in operand layout (all 64 lanes convert, then lanes read their
// operands), so no cross-wavefront synchronisation is needed until the four
// partial tiles are added in a fixed order at the end (deterministic).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRows = 16;     // output rows per workgroup (MFMA N)
constexpr int kChunk = 4;     // blocks converted per LDS round

// LDS of one wavefront's activation operands for a chunk, MT tokens:
//   hi / lo: [kChunk][8 steps][4 lane groups][MT] x 8 halves (16 B per entry)
//   xs_hi / xs_lo: [kChunk][4 lane groups][MT] two halves (X_{2g}, X_{2g+1})
//   shift: [kChunk][16] exponent sh per token (entries >= MT unused)
template <int MT>
struct WaveLds {
  static constexpr int kOp = kChunk * 8 * 4 * MT;
  uint4 hi[kOp];
  uint4 lo[kOp];
  uint32_t xs_hi[kChunk * 4 * MT];
  uint32_t xs_lo[kChunk * 4 * MT];
  int shift[kChunk * 16];
};

template <int MT, bool GU>
struct Lds {
  union {
    WaveLds<MT> wave[kWaves];
    float red[GU ? 2 : 1][kWaves][16][kRows];
  };
};

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

__device__ __forceinline__ uint32_t pack_half2(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Exponent that maps a block maximum into [2^14, 2^15) (0 for an all-zero
// block).
__device__ __forceinline__ int block_shift(float amax) {
  const int eb = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  return amax > 0.0f ? 141 - eb : 0;
}

// v = hi + lo with binary16 halves, to 22 significant bits.
__device__ __forceinline__ void split_half(float v, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(v);
  lo = static_cast<_Float16>(v - static_cast<float>(hi));
}

// Converts this wavefront's activations of blocks [b0, b0 + nb) into operand
// layout.  Lane l owns values 4l .. 4l+3 of each 256-block: operand step
// s = (l % 16) / 2, lane group g = l / 16, halves 4*(l%2) .. +3, sub-block
// j = l / 8.
template <int MT, bool BF16>
__device__ __forceinline__ void convert_chunk(WaveLds<MT>& L, const void* __restrict__ x,
                                              const int* xrow, int ldx, int mt, int b0, int nb,
                                              int lane) {
  const int s = (lane & 15) >> 1;
  const int g = lane >> 4;
  const int half = lane & 1;
  for (int t = 0; t < MT; ++t) {
    if (t >= mt) break;
    for (int bi = 0; bi < nb; ++bi) {
      const float4 v = load_x4<BF16>(x, static_cast<size_t>(xrow[t]) * ldx +
                                            static_cast<size_t>(b0 + bi) * kQK + 4 * lane);
      float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
      amax = wave_max(amax);
      const int sh = block_shift(amax);
      const float v0 = ldexpf(v.x, sh), v1 = ldexpf(v.y, sh);
      const float v2 = ldexpf(v.z, sh), v3 = ldexpf(v.w, sh);
      _Float16 h0, h1, h2, h3, l0, l1, l2, l3;
      split_half(v0, h0, l0);
      split_half(v1, h1, l1);
      split_half(v2, h2, l2);
      split_half(v3, h3, l3);
      const int e = ((bi * 8 + s) * 4 + g) * MT + t;
      reinterpret_cast<uint2*>(&L.hi[e])[half] = make_uint2(pack_half2(h0, h1), pack_half2(h2, h3));
      reinterpret_cast<uint2*>(&L.lo[e])[half] = make_uint2(pack_half2(l0, l1), pack_half2(l2, l3));
      // sum of the scaled values of sub-block j = lane / 8 (eight lanes)
      float xs = (v0 + v1) + (v2 + v3);
      xs += __shfl_xor(xs, 1, 64);
      xs += __shfl_xor(xs, 2, 64);
      xs += __shfl_xor(xs, 4, 64);
      if ((lane & 7) == 0) {
        const int j = lane >> 3;  // sub-block: lane group j/2, K slot j%2
        // |xs| < 32 * 2^15; the sum is stored as xs * 2^-6 (the mins are
        // used as m * 2^6 <= 4032, still exact) to stay inside binary16
        _Float16 xh, xl;
        split_half(xs * 0.015625f, xh, xl);
        const int ei = (bi * 4 + (j >> 1)) * MT + t;
        reinterpret_cast<uint16_t*>(&L.xs_hi[ei])[j & 1] = __builtin_bit_cast(uint16_t, xh);
        reinterpret_cast<uint16_t*>(&L.xs_lo[ei])[j & 1] = __builtin_bit_cast(uint16_t, xl);
      }
      if (lane == 0) L.shift[bi * 16 + t] = sh;
    }
  }
}

// Eight quants (low nibbles of the two dwords) times sc as binary16: a byte
// permute builds 1024 + q and one fused (1024 + q) * sc - 1024 * sc per pair
// yields q * sc exactly.
__device__ __forceinline__ v8h weights8(uint32_t w0, uint32_t w1, v2h s, v2h o) {
  const uint32_t k64 = 0x64646464u;
  const uint32_t m0 = w0 & 0x0F0F0F0Fu, m1 = w1 & 0x0F0F0F0Fu;
  const v2h p0 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m0, 0x04010400u));
  const v2h p1 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m0, 0x04030402u));
  const v2h p2 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m1, 0x04010400u));
  const v2h p3 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m1, 0x04030402u));
  const v2h r0 = __builtin_elementwise_fma(p0, s, o);
  const v2h r1 = __builtin_elementwise_fma(p1, s, o);
  const v2h r2 = __builtin_elementwise_fma(p2, s, o);
  const v2h r3 = __builtin_elementwise_fma(p3, s, o);
  return v8h{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

struct BlockRegs {
  uint4 h;   // header
  uint4 q0;  // quant bytes 32g .. 32g+15
  uint4 q1;  // quant bytes 32g+16 .. 32g+31
};

__device__ __forceinline__ void load_block(const uint8_t* __restrict__ blk, int g, BlockRegs& r) {
  r.h = *reinterpret_cast<const uint4*>(blk);
  r.q0 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * g);
  r.q1 = *reinterpret_cast<const uint4*>(blk + 32 + 32 * g);
}

// One block of one matrix: the main chain (cm) and the min term (cn).
template <int MT>
__device__ __forceinline__ void block_mfma(const BlockRegs& r, int g, const WaveLds<MT>& L, int bi,
                                           int tok, bool active, float& d, float& dmin,
                                           v4f& cm, v4f& cn) {
  d = half_bits_to_float(r.h.x & 0xFFFFu);
  dmin = half_bits_to_float(r.h.x >> 16);
  uint32_t sc0, mn0, sc1, mn1;
  scale_min_rt(r.h, 2 * g, sc0, mn0);
  scale_min_rt(r.h, 2 * g + 1, sc1, mn1);
  const _Float16 fs0 = static_cast<_Float16>(static_cast<float>(sc0));
  const _Float16 fs1 = static_cast<_Float16>(static_cast<float>(sc1));
  const _Float16 fo0 = static_cast<_Float16>(-1024.0f * static_cast<float>(sc0));
  const _Float16 fo1 = static_cast<_Float16>(-1024.0f * static_cast<float>(sc1));
  const v2h s0 = v2h{fs0, fs0}, o0 = v2h{fo0, fo0};
  const v2h s1 = v2h{fs1, fs1}, o1 = v2h{fo1, fo1};
  const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
  cm = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const v8h b = s < 4 ? weights8(w[2 * s], w[2 * s + 1], s0, o0)
                        : weights8(w[2 * (s - 4)] >> 4, w[2 * (s - 4) + 1] >> 4, s1, o1);
    v8h ah = v8h{0, 0, 0, 0, 0, 0, 0, 0}, al = ah;
    if (active) {
      const int e = ((bi * 8 + s) * 4 + g) * MT + tok;
      ah = __builtin_bit_cast(v8h, L.hi[e]);
      al = __builtin_bit_cast(v8h, L.lo[e]);
    }
    cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, b, cm, 0, 0, 0);
    cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b, cm, 0, 0, 0);
  }
  // min term: K slots 0 and 1 of lane group g hold (m_{2g}, m_{2g+1}) and the
  // activation sums (X_{2g}, X_{2g+1}); the other slots are zero
  const v8h bm = v8h{static_cast<_Float16>(64.0f * static_cast<float>(mn0)),
                     static_cast<_Float16>(64.0f * static_cast<float>(mn1)), 0, 0, 0, 0, 0, 0};
  v8h xh = v8h{0, 0, 0, 0, 0, 0, 0, 0}, xl = xh;
  if (active) {
    const v2h ph = __builtin_bit_cast(v2h, L.xs_hi[(bi * 4 + g) * MT + tok]);
    const v2h pl = __builtin_bit_cast(v2h, L.xs_lo[(bi * 4 + g) * MT + tok]);
    xh[0] = ph[0]; xh[1] = ph[1];
    xl[0] = pl[0]; xl[1] = pl[1];
  }
  cn = v4f{0.f, 0.f, 0.f, 0.f};
  cn = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bm, cn, 0, 0, 0);
  cn = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, bm, cn, 0, 0, 0);
}

__device__ __forceinline__ void lds_fence() {
  // this wavefront's LDS writes complete before its later LDS reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int MT, bool GU, bool BF16>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(GemvArgs a) {
  __shared__ Lds<MT, GU> lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = a.k / kQK;

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

  const int n0 = blockIdx.x * kRows;
  const int nl = lane & 15;   // B operand weight row / A operand token / C row-slot
  const int g = lane >> 4;    // lane group: K slots 8g .. 8g+7
  const int row = min(n0 + nl, a.n - 1);
  const size_t row_off = static_cast<size_t>(row) * K * kBlockBytes;
  const uint8_t* wg = a.w + static_cast<size_t>(expert) * a.mat_bytes + row_off;
  const uint8_t* wu = GU ? a.w_up + static_cast<size_t>(expert) * a.mat_bytes + row_off : nullptr;

  const int kb0 = (wave * K) / kWaves;
  const int kb1 = ((wave + 1) * K) / kWaves;
  const bool active = nl < mt;  // the A operand token of this lane exists

  float yg[4] = {0.f, 0.f, 0.f, 0.f};
  float yu[4] = {0.f, 0.f, 0.f, 0.f};
  WaveLds<MT>& L = lds.wave[wave];

  for (int cb = kb0; cb < kb1; cb += kChunk) {
    const int nb = min(kChunk, kb1 - cb);
    // issue every weight load of the chunk before converting activations
    BlockRegs rg[kChunk], ru[kChunk];
#pragma unroll
    for (int bi = 0; bi < kChunk; ++bi) {
      if (bi < nb) {
        load_block(wg + static_cast<size_t>(cb + bi) * kBlockBytes, g, rg[bi]);
        if constexpr (GU) load_block(wu + static_cast<size_t>(cb + bi) * kBlockBytes, g, ru[bi]);
      }
    }
    convert_chunk<MT, BF16>(L, a.x, xrow, a.ldx, mt, cb, nb, lane);
    lds_fence();
#pragma unroll
    for (int bi = 0; bi < kChunk; ++bi) {
      if (bi < nb) {
        const int4 shv = *reinterpret_cast<const int4*>(&L.shift[bi * 16 + 4 * g]);
        const int shs[4] = {shv.x, shv.y, shv.z, shv.w};
        float d, dmin;
        v4f cm, cn;
        block_mfma<MT>(rg[bi], g, L, bi, nl, active, d, dmin, cm, cn);
#pragma unroll
        for (int i = 0; i < 4; ++i) yg[i] += ldexpf(fmaf(d, cm[i], -dmin * cn[i]), -shs[i]);
        if constexpr (GU) {
          block_mfma<MT>(ru[bi], g, L, bi, nl, active, d, dmin, cm, cn);
#pragma unroll
          for (int i = 0; i < 4; ++i) yu[i] += ldexpf(fmaf(d, cm[i], -dmin * cn[i]), -shs[i]);
        }
      }
    }
    lds_fence();
  }

  __syncthreads();
  // C layout: lane holds tokens 4g .. 4g+3 of weight row nl
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lds.red[0][wave][4 * g + i][nl] = yg[i];
    if constexpr (GU) lds.red[GU ? 1 : 0][wave][4 * g + i][nl] = yu[i];
  }
  __syncthreads();
  const int t = tid / kRows;
  const int r = tid % kRows;
  if (t < mt && n0 + r < a.n) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += lds.red[0][w][t][r];
    float out = s;
    if constexpr (GU) {
      float su = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) su += lds.red[GU ? 1 : 0][w][t][r];
      out = silu_mul(s, su);
    }
    a.y[static_cast<size_t>(yrow[t]) * a.ldy + n0 + r] = out;
  }
}

template <int MT>
hipError_t dispatch_m(const GemvArgs& a, hipStream_t stream) {
  const dim3 grid((a.n + kRows - 1) / kRows, a.slot_expert ? a.slots : 1);
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
  if (gu) {
    if (bf) gemv_mfma_kernel<MT, true, true><<<grid, dim3(kThreads), 0, stream>>>(a);
    else gemv_mfma_kernel<MT, true, false><<<grid, dim3(kThreads), 0, stream>>>(a);
  } else {
    if (bf) gemv_mfma_kernel<MT, false, true><<<grid, dim3(kThreads), 0, stream>>>(a);
    else gemv_mfma_kernel<MT, false, false><<<grid, dim3(kThreads), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t stream) {
  switch (a.m) {
    case 1: return dispatch_m<1>(a, stream);
    case 2: return dispatch_m<2>(a, stream);
    case 3: return dispatch_m<3>(a, stream);
    case 4: return dispatch_m<4>(a, stream);
    case 5: return dispatch_m<5>(a, stream);
    case 6: return dispatch_m<6>(a, stream);
    case 7: return dispatch_m<7>(a, stream);
    default: return dispatch_m<8>(a, stream);
  }
}

}  // namespace q4k
