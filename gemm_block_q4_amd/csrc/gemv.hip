// Dequant-fused Q4_K GEMV for the decode regime (1..8 tokens), gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k; "realizar -- ffn.rs",
// fused_ffn_swiglu_gpu: gate and up GEMVs, silu(gate) * up, then the down
// GEMV.  Here the gate and up GEMVs run in one pass over both matrices and
// the silu * mul is applied before the single store.
//
// Work decomposition.  A workgroup (4 wavefronts) owns `rows` consecutive
// output rows; every (row, 256-block) pair is one work item and one lane
// processes one whole block (the 144 bytes are contiguous, and consecutive
// lanes take consecutive blocks, so a wavefront's loads cover one contiguous
// run of 64 * 144 bytes).  The activations of the slot's tokens are staged
// once per workgroup in LDS (padded by 16 bytes per 256 values so that lanes
// reading different blocks hit different banks) together with the sum of
// every 32-value sub-block, which turns the min term into one FMA per
// sub-block:
//   sum_i w_i x_i = d*sc_j * sum_i q_i x_i - dmin*m_j * sum_i x_i.
// Each item leaves one partial per token in LDS; a final pass adds the k/256
// partials of a row in order (deterministic) and stores y or silu(g)*u.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

constexpr int kThreads = 256;
constexpr int kXPad = 260;   // floats per staged 256-value block

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

__device__ __forceinline__ float dot4_nibbles(uint32_t packed, float4 xv, float acc) {
  // packed holds four bytes whose values are the quants (low nibbles) or
  // 16 * quants (high nibbles masked in place).
  // (byte extract + int->float is selected as v_cvt_f32_ubyteN)
  acc = fmaf(static_cast<float>(packed & 0xFFu), xv.x, acc);
  acc = fmaf(static_cast<float>((packed >> 8) & 0xFFu), xv.y, acc);
  acc = fmaf(static_cast<float>((packed >> 16) & 0xFFu), xv.z, acc);
  acc = fmaf(static_cast<float>(packed >> 24), xv.w, acc);
  return acc;
}

// Adds one block's contribution for every token to acc[].
template <int M, bool XLDS, bool BF16>
__device__ __forceinline__ void block_dot(const uint4* __restrict__ blk, const float* xs,
                                          const float* xsum, const void* __restrict__ xg,
                                          const int* xrow, int ldx, int b, int nsub,
                                          float (&acc)[M]) {
  const uint4 h = blk[0];
  uint4 q[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) q[c] = blk[1 + c];
  const float d = half_bits_to_float(h.x & 0xFFFFu);
  const float dmin = half_bits_to_float(h.x >> 16);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t sc0, mn0, sc1, mn1;
    switch (g) {
      case 0: scale_min<0>(h, sc0, mn0); scale_min<1>(h, sc1, mn1); break;
      case 1: scale_min<2>(h, sc0, mn0); scale_min<3>(h, sc1, mn1); break;
      case 2: scale_min<4>(h, sc0, mn0); scale_min<5>(h, sc1, mn1); break;
      default: scale_min<6>(h, sc0, mn0); scale_min<7>(h, sc1, mn1); break;
    }
    const float s0 = d * static_cast<float>(sc0);
    const float s1 = d * static_cast<float>(sc1) * 0.0625f;  // high nibbles read as 16*q
    const float m0 = dmin * static_cast<float>(mn0);
    const float m1 = dmin * static_cast<float>(mn1);
    const uint32_t w8[8] = {q[2 * g].x, q[2 * g].y, q[2 * g].z, q[2 * g].w,
                            q[2 * g + 1].x, q[2 * g + 1].y, q[2 * g + 1].z, q[2 * g + 1].w};
    float lo[M], hi[M];
#pragma unroll
    for (int t = 0; t < M; ++t) { lo[t] = 0.f; hi[t] = 0.f; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wl = w8[i] & 0x0F0F0F0Fu;
      const uint32_t wh = w8[i] & 0xF0F0F0F0u;
#pragma unroll
      for (int t = 0; t < M; ++t) {
        float4 xl, xh;
        if constexpr (XLDS) {
          const float* base = xs + (t * nsub / 8 + b) * kXPad + 64 * g + 4 * i;
          xl = *reinterpret_cast<const float4*>(base);
          xh = *reinterpret_cast<const float4*>(base + 32);
        } else {
          const size_t base = static_cast<size_t>(xrow[t]) * ldx + b * kQK + 64 * g + 4 * i;
          xl = load_x4<BF16>(xg, base);
          xh = load_x4<BF16>(xg, base + 32);
        }
        lo[t] = dot4_nibbles(wl, xl, lo[t]);
        hi[t] = dot4_nibbles(wh, xh, hi[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const float* xsum_t = xsum + t * nsub + b * 8 + 2 * g;
      float a = acc[t];
      a = fmaf(s0, lo[t], a);
      a = fmaf(s1, hi[t], a);
      a = fmaf(-m0, xsum_t[0], a);
      a = fmaf(-m1, xsum_t[1], a);
      acc[t] = a;
    }
  }
}

template <int M, bool GU, bool XLDS, bool BF16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a, int rows_per_wg) {
  extern __shared__ float smem[];
  const int K = a.k / kQK;
  const int nsub = a.k / kSub;
  const int tid = threadIdx.x;

  // Slot: dense mode has one slot holding tokens 0..m-1 of expert 0.
  int expert = 0, mt = a.m;
  int xrow[M], yrow[M];
  if (a.slot_expert != nullptr) {
    const int slot = blockIdx.y;
    expert = a.slot_expert[slot];
    if (expert < 0) return;  // uniform over the workgroup
    mt = min(a.slot_count[slot], M);
#pragma unroll
    for (int t = 0; t < M; ++t) {
      xrow[t] = t < mt ? a.slot_x[slot * kMaxTokens + t] : 0;
      yrow[t] = t < mt ? a.slot_y[slot * kMaxTokens + t] : 0;
    }
  } else {
#pragma unroll
    for (int t = 0; t < M; ++t) {
      xrow[t] = t < mt ? t : 0;
      yrow[t] = t;
    }
  }
  const uint8_t* wg = a.w + static_cast<size_t>(expert) * a.mat_bytes;
  const uint8_t* wu = GU ? a.w_up + static_cast<size_t>(expert) * a.mat_bytes : nullptr;

  const int row0 = blockIdx.x * rows_per_wg;
  const int rows = min(rows_per_wg, a.n - row0);
  const int items = rows * K;

  // LDS: [xs: M*K*kXPad if XLDS][xsum: M*nsub][partials: (GU?2:1)*M*items]
  float* xs = smem;
  float* xsum = smem + (XLDS ? M * K * kXPad : 0);
  float* part = xsum + M * nsub;

  // Stage activations (tokens beyond mt read as zero).
  if constexpr (XLDS) {
    const int groups = M * a.k / 4;
    for (int i = tid; i < groups; i += kThreads) {
      const int t = (i * 4) / a.k;
      const int col = (i * 4) % a.k;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < mt) v = load_x4<BF16>(a.x, static_cast<size_t>(xrow[t]) * a.ldx + col);
      *reinterpret_cast<float4*>(xs + (t * K + col / kQK) * kXPad + col % kQK) = v;
    }
    __syncthreads();
  }
  // Sub-block sums of the activations.
  for (int i = tid; i < M * nsub; i += kThreads) {
    const int t = i / nsub;
    const int j = i % nsub;
    float s = 0.f;
    if (t < mt) {
#pragma unroll
      for (int c = 0; c < kSub; c += 4) {
        float4 v;
        if constexpr (XLDS) {
          v = *reinterpret_cast<const float4*>(xs + (t * K + j / 8) * kXPad + (j % 8) * kSub + c);
        } else {
          v = load_x4<BF16>(a.x, static_cast<size_t>(xrow[t]) * a.ldx + j * kSub + c);
        }
        s += (v.x + v.y) + (v.z + v.w);
      }
    }
    xsum[i] = s;
  }
  __syncthreads();

  for (int item = tid; item < items; item += kThreads) {
    const int r = item / K;
    const int b = item % K;
    const size_t boff = (static_cast<size_t>(row0 + r) * K + b) * kBlockBytes;
    float acc[M];
#pragma unroll
    for (int t = 0; t < M; ++t) acc[t] = 0.f;
    block_dot<M, XLDS, BF16>(reinterpret_cast<const uint4*>(wg + boff), xs, xsum, a.x, xrow,
                             a.ldx, b, nsub, acc);
#pragma unroll
    for (int t = 0; t < M; ++t) part[t * items + item] = acc[t];
    if constexpr (GU) {
#pragma unroll
      for (int t = 0; t < M; ++t) acc[t] = 0.f;
      block_dot<M, XLDS, BF16>(reinterpret_cast<const uint4*>(wu + boff), xs, xsum, a.x, xrow,
                               a.ldx, b, nsub, acc);
#pragma unroll
      for (int t = 0; t < M; ++t) part[(M + t) * items + item] = acc[t];
    }
  }
  __syncthreads();

  // Row totals in block order; tokens past mt are not stored.
  for (int i = tid; i < rows * M; i += kThreads) {
    const int t = i / rows;
    const int r = i % rows;
    if (t >= mt) continue;
    float s = 0.f;
    for (int b = 0; b < K; ++b) s += part[t * items + r * K + b];
    float out = s;
    if constexpr (GU) {
      float su = 0.f;
      for (int b = 0; b < K; ++b) su += part[(M + t) * items + r * K + b];
      out = silu_mul(s, su);
    }
    a.y[static_cast<size_t>(yrow[t]) * a.ldy + row0 + r] = out;
  }
}

template <int M, bool GU, bool XLDS, bool BF16>
hipError_t launch_one(const GemvArgs& a, int rows_per_wg, size_t lds, hipStream_t stream) {
  const dim3 grid((a.n + rows_per_wg - 1) / rows_per_wg, a.slot_expert ? a.slots : 1);
  auto kern = gemv_kernel<M, GU, XLDS, BF16>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  kern<<<grid, dim3(kThreads), lds, stream>>>(a, rows_per_wg);
  return hipGetLastError();
}

template <int M>
hipError_t dispatch_m(const GemvArgs& a, int rows_per_wg, hipStream_t stream) {
  const int K = a.k / kQK;
  const int nsub = a.k / kSub;
  const int parts = (a.w_up ? 2 : 1) * M * rows_per_wg * K;
  const size_t base = static_cast<size_t>(M * nsub + parts) * sizeof(float);
  const size_t xlds = static_cast<size_t>(M) * K * kXPad * sizeof(float);
  const bool use_lds = base + xlds <= 64 * 1024;
  const size_t lds = base + (use_lds ? xlds : 0);
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
#define Q4K_GEMV_CASE(GUV, XL, BFV) \
  if (gu == GUV && use_lds == XL && bf == BFV) return launch_one<M, GUV, XL, BFV>(a, rows_per_wg, lds, stream);
  Q4K_GEMV_CASE(false, true, false)
  Q4K_GEMV_CASE(false, true, true)
  Q4K_GEMV_CASE(false, false, false)
  Q4K_GEMV_CASE(false, false, true)
  Q4K_GEMV_CASE(true, true, false)
  Q4K_GEMV_CASE(true, true, true)
  Q4K_GEMV_CASE(true, false, false)
  Q4K_GEMV_CASE(true, false, true)
#undef Q4K_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  // Rows per workgroup: enough workgroups to fill 256 CUs twice over, and a
  // bounded partial-sum area in LDS.
  const int K = a.k / kQK;
  int rows = a.n / 512;
  rows = rows < 1 ? 1 : (rows > 16 ? 16 : rows);
  while (rows > 1 && rows * K > 1024) --rows;
  switch (a.m) {
    case 1: return dispatch_m<1>(a, rows, stream);
    case 2: return dispatch_m<2>(a, rows, stream);
    case 3: return dispatch_m<3>(a, rows, stream);
    case 4: return dispatch_m<4>(a, rows, stream);
    case 5: return dispatch_m<5>(a, rows, stream);
    case 6: return dispatch_m<6>(a, rows, stream);
    case 7: return dispatch_m<7>(a, rows, stream);
    default: return dispatch_m<8>(a, rows, stream);
  }
}

}  // namespace q4k
