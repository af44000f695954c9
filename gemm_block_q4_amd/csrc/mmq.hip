// Q8_1 x Q4_K integer GEMM (MMQ) for the prefill regime, gfx950 int8 MFMA.
//
// "spark_model/layers/ops/q4k_mmq.rs", q4k_mmq_gemm: C[m,n] = A_q8[m,k] x
// W_q4k[n,k]^T; "realizar -- ffn.rs", fused_ffn_swiglu_gpu_true_dp4a: the
// integer dot comes first and the scales are applied afterwards.  For token
// t, weight row n and 32-value sub-block j:
//   P = sum_{i<32} q_w * q_a                       (v_mfma_i32_32x32x32_i8)
//   y += d_a[t,j] * ((d*sc_j)[n] * P - (dmin*m_j)[n] * S[t,j])
// where S is the integer block sum stored with the activation scale.  One
// 32x32x32 MFMA covers exactly one sub-block, so its int32 result is the
// per-sub-block partial P (the test hook writes it out unchanged).
//
// Tiling: a workgroup of four wavefronts computes 64 tokens x 64 weight rows;
// wavefront (wm, wn) owns the 32 x 32 sub-tile.  For every 256-wide k block
// the workgroup stages the 64 x 256 activation quants and their 64 x 8 scale
// words in LDS; each lane reads its weight row's quants straight from global
// memory (16 contiguous bytes = 16 low-nibble weights of sub-block 2g and 16
// high-nibble weights of sub-block 2g+1) and widens the nibbles to int8 in
// registers.  With w_up set the same activations feed the gate and the up
// rows and the epilogue stores h = silu(g) * u.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 64;
constexpr int kBN = 64;
constexpr int kArow = kQK + 16;  // padded LDS row of activation quants (bytes)

struct WeightLane {
  v4i lo[4];   // sub-blocks 0,2,4,6: 16 int8 weights each
  v4i hi[4];   // sub-blocks 1,3,5,7
  float sw[8]; // d * sc_j
  float mw[8]; // dmin * m_j
};

__device__ __forceinline__ void load_weight_lane(const uint8_t* __restrict__ blk, int kg,
                                                 WeightLane& wl) {
  const uint4 h = *reinterpret_cast<const uint4*>(blk);
  const float d = half_bits_to_float(h.x & 0xFFFFu);
  const float dmin = half_bits_to_float(h.x >> 16);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint4 v = *reinterpret_cast<const uint4*>(blk + 16 + 32 * g + 16 * kg);
    wl.lo[g] = v4i{static_cast<int>(v.x & 0x0F0F0F0Fu), static_cast<int>(v.y & 0x0F0F0F0Fu),
                   static_cast<int>(v.z & 0x0F0F0F0Fu), static_cast<int>(v.w & 0x0F0F0F0Fu)};
    wl.hi[g] = v4i{static_cast<int>((v.x >> 4) & 0x0F0F0F0Fu), static_cast<int>((v.y >> 4) & 0x0F0F0F0Fu),
                   static_cast<int>((v.z >> 4) & 0x0F0F0F0Fu), static_cast<int>((v.w >> 4) & 0x0F0F0F0Fu)};
  }
  uint32_t sc, mn;
#define Q4K_SM(S) scale_min<S>(h, sc, mn); wl.sw[S] = d * static_cast<float>(sc); wl.mw[S] = dmin * static_cast<float>(mn);
  Q4K_SM(0) Q4K_SM(1) Q4K_SM(2) Q4K_SM(3) Q4K_SM(4) Q4K_SM(5) Q4K_SM(6) Q4K_SM(7)
#undef Q4K_SM
}

template <bool GU, bool PARTIALS>
__global__ __launch_bounds__(256) void mmq_kernel(MmqArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t sA[kBM * kArow];
  __shared__ __attribute__((aligned(16))) float sD[8][kBM];   // activation scale d_a per (sub-block, token)
  __shared__ __attribute__((aligned(16))) float sS[8][kBM];   // d_a * S per (sub-block, token)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int K = a.k / kQK;
  const int nsub = a.k / kSub;

  // This lane's weight row (clamped for the ragged edge; results discarded).
  const int nrow = n0 + wn * 32 + (lane & 31);
  const int nrow_c = min(nrow, a.n - 1);
  const int kg = lane >> 5;  // which 16 of the 32 k values of a sub-block
  const uint8_t* wrow = a.w + static_cast<size_t>(nrow_c) * K * kBlockBytes;
  const uint8_t* urow = GU ? a.w_up + static_cast<size_t>(nrow_c) * K * kBlockBytes : nullptr;

  v16i zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0;
  float acc[16], accu[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) { acc[i] = 0.f; accu[i] = 0.f; }

  for (int b = 0; b < K; ++b) {
    // Stage activation quants: 64 tokens x 256 bytes, 64 bytes per thread.
    {
      const int tok = tid >> 2;
      const int part = tid & 3;
      const int tg = t0 + tok;
      uint4 v[4];
      if (tg < a.m) {
        const uint4* src = reinterpret_cast<const uint4*>(a.qs + static_cast<size_t>(tg) * a.k + b * kQK + part * 64);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = src[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(sA + tok * kArow + part * 64 + c * 16) = v[c];
    }
    // Stage activation scales: 64 tokens x 8 words.
    for (int i = tid; i < kBM * 8; i += 256) {
      const int tok = i >> 3;
      const int j = i & 7;
      const int tg = t0 + tok;
      float dv = 0.f, sv = 0.f;
      if (tg < a.m) {
        const uint32_t w = a.ds[static_cast<size_t>(tg) * nsub + b * 8 + j];
        dv = half_bits_to_float(w & 0xFFFFu);
        sv = dv * static_cast<float>(static_cast<int16_t>(w >> 16));  // exact in binary32
      }
      sD[j][tok] = dv;
      sS[j][tok] = sv;
    }
    __syncthreads();

    WeightLane wgt, wup;
    load_weight_lane(wrow + b * kBlockBytes, kg, wgt);
    if constexpr (GU) load_weight_lane(urow + b * kBlockBytes, kg, wup);

    const int arow = wm * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v4i av = *reinterpret_cast<const v4i*>(sA + arow * kArow + j * 32 + kg * 16);
      const v4i bv = (j & 1) ? wgt.hi[j >> 1] : wgt.lo[j >> 1];
      const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zero, 0, 0, 0);
      v16i pu;
      if constexpr (GU) {
        const v4i uv = (j & 1) ? wup.hi[j >> 1] : wup.lo[j >> 1];
        pu = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, uv, zero, 0, 0, 0);
      }
      if constexpr (PARTIALS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tl = wm * 32 + 8 * (i >> 2) + 4 * kg + (i & 3);
          const int tg = t0 + tl;
          if (tg < a.m && nrow < a.n)
            a.partials[(static_cast<size_t>(tg) * a.n + nrow) * nsub + b * 8 + j] = p[i];
        }
      } else {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int tl = wm * 32 + 8 * i4 + 4 * kg;
          const float4 dv = *reinterpret_cast<const float4*>(&sD[j][tl]);
          const float4 sv = *reinterpret_cast<const float4*>(&sS[j][tl]);
          const float da[4] = {dv.x, dv.y, dv.z, dv.w};
          const float sa[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * i4 + r;
            float v = fmaf(wgt.sw[j], static_cast<float>(p[i]) * da[r], acc[i]);
            acc[i] = fmaf(-wgt.mw[j], sa[r], v);
            if constexpr (GU) {
              float vu = fmaf(wup.sw[j], static_cast<float>(pu[i]) * da[r], accu[i]);
              accu[i] = fmaf(-wup.mw[j], sa[r], vu);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if constexpr (!PARTIALS) {
    if (nrow < a.n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tg = t0 + wm * 32 + 8 * (i >> 2) + 4 * kg + (i & 3);
        if (tg < a.m) {
          float out = acc[i];
          if constexpr (GU) out = silu_mul(acc[i], accu[i]);
          a.y[static_cast<size_t>(tg) * a.n + nrow] = out;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_mmq(const MmqArgs& a, hipStream_t stream) {
  const dim3 grid((a.n + kBN - 1) / kBN, (a.m + kBM - 1) / kBM);
  if (a.partials)
    mmq_kernel<false, true><<<grid, dim3(256), 0, stream>>>(a);
  else if (a.w_up)
    mmq_kernel<true, false><<<grid, dim3(256), 0, stream>>>(a);
  else
    mmq_kernel<false, false><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace q4k
