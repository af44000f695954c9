// Per-row FP8 (E4M3) prefill recipe, gfx950.
//
// "aprender-serve -- cublas_prefill/fp8_recipe.rs": every activation row
// (token) and every weight row (output channel) gets its own scale
// 448/absmax (fp8_absmax_rows, fp8_quantize_rows: E4M3 with round to nearest
// even, saturating at 448, subnormals kept); the GEMM of the two FP8 matrices
// writes D in BF16 with alpha 1; the per-row scales are applied after it
// (fp8_dequant_outer): Y[t, c] = D[t, c] * (a[t]/448) * (w[c]/448), an
// all-zero row's absmax taken as 1.
//
// E4M3 is the OCP E4M3FN format (bias 7, largest finite 448, no infinity),
// the format gfx950's FP8 matrix instructions read.  The GEMM runs on
// v_mfma_f32_32x32x64_f8f6f4 (exact products, f32 accumulation); its
// epilogue rounds D to BF16 as the page's GEMM output is and then applies the
// two outer scales, so D never goes to memory.
#include <hip/hip_runtime.h>

#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kE4m3Max = 448.f;

// --- row absmax ---------------------------------------------------------------

// One workgroup of 256 threads per row; VEC: 16-byte reads (cols % 4 == 0,
// 16-byte aligned rows).  Max over the wavefront, then over the four
// wavefronts in LDS.
template <bool VEC>
__global__ __launch_bounds__(256) void absmax_rows_kernel(const float* __restrict__ x, int cols,
                                                          float* __restrict__ absmax) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const float* xr = x + static_cast<size_t>(row) * cols;
  float m = 0.f;
  if constexpr (VEC) {
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    for (int i = threadIdx.x; i < cols / 4; i += 256) {
      const float4 v = x4[i];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  } else {
    for (int i = threadIdx.x; i < cols; i += 256) m = fmaxf(m, fabsf(xr[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) absmax[row] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

// --- E4M3 encoding ---------------------------------------------------------------

// E4M3FN code of a finite v: the nearest value, ties to even, |v| saturated
// at 448.  Below 2^-6 the subnormal code rint(|v| * 2^9) (0..8, where 8 is
// the smallest normal's code); from 2^-6 up, the binary32 exponent rebiased
// from 127 to 7 and the mantissa cut to three bits with round to nearest
// even, a carry out of the mantissa moving to the next exponent.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fminf(fabsf(v), kE4m3Max);
  const uint32_t sub = static_cast<uint32_t>(rintf(a * 512.f));
  const uint32_t b = __float_as_uint(a);
  uint32_t e = (b >> 23) - 120u;
  uint32_t m3 = (b >> 20) & 7u;
  const uint32_t rbit = (b >> 19) & 1u;
  const uint32_t sticky = b & 0x7FFFFu;
  m3 += rbit & ((sticky != 0u) | (m3 & 1u));
  e += m3 >> 3;
  m3 &= 7u;
  return sign | (a < 0.015625f ? sub : (e << 3) | m3);
}

__device__ __forceinline__ float row_scale(const float* absmax, int row) {
  const float am = absmax[row];
  return kE4m3Max / (am == 0.f ? 1.f : am);  // correctly rounded binary32 quotient
}

// VEC: sixteen consecutive values of a row per thread (cols % 16 == 0,
// 16-byte aligned x and q); otherwise one value per thread.
template <bool VEC>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ x, const float* __restrict__ absmax,
                                                            int cols, size_t units, uint8_t* __restrict__ q) {
  const size_t u = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (u >= units) return;
  if constexpr (VEC) {
    const size_t base = u * 16;
    const float scale = row_scale(absmax, static_cast<int>(base / static_cast<size_t>(cols)));
    const float4* xs = reinterpret_cast<const float4*>(x + base);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = xs[i];
      w[i] = e4m3_code(v.x * scale) | e4m3_code(v.y * scale) << 8 | e4m3_code(v.z * scale) << 16 |
             e4m3_code(v.w * scale) << 24;
    }
    *reinterpret_cast<uint4*>(q + base) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    const float scale = row_scale(absmax, static_cast<int>(u / static_cast<size_t>(cols)));
    q[u] = static_cast<uint8_t>(e4m3_code(x[u] * scale));
  }
}

// --- FP8 GEMM with the outer dequant ----------------------------------------------------

constexpr int kFBN = 128;           // weight rows per workgroup (two wavefront columns of 64)
constexpr int kFK = 128;            // k bytes per stage
constexpr int kFStride = kFK + 16;  // LDS row stride in bytes: b128 reads of 16 rows hit distinct banks

template <int WM>
struct FStage {
  uint8_t a[64 * WM * kFStride];  // activation codes [token][k]
  uint8_t w[kFBN * kFStride];     // weight codes [row][k]
};

// Workgroup tile: 64 WM tokens x 128 weight rows, 2 WM wavefronts, each
// 64 tokens x 64 rows as 2 x 2 tiles of 32 x 32.  Tokens are the MFMA A
// operand (rows of C) and weight rows the B operand (columns of C), so lane l
// holds weight row l % 32 of its tile and a wavefront's stores cover runs of
// consecutive y columns.  Within one 64-deep MFMA step a lane supplies the 32
// k values 32 (l / 32) .. +31 of its A row and its B row (the instruction
// pairs A and B bytes by the same lane half and byte position).
// Staging: k advances by 128 per stage through two LDS buffers; the global
// loads of stages s + 1 and s + 2 are in flight in two register sets while
// stage s is multiplied.  Tokens past
// m, weight rows past n and k past the end read zeros (raw buffer bounds and
// kOob offsets), which add nothing.
template <int WM>
__global__ __launch_bounds__(128 * WM) void fp8_gemm_kernel(const uint8_t* __restrict__ a,
                                                            const float* __restrict__ a_absmax,
                                                            const uint8_t* __restrict__ w,
                                                            const float* __restrict__ w_absmax,
                                                            float* __restrict__ y, int m, int n, int k) {
  constexpr int kThreads = 128 * WM;
  constexpr int kBM = 64 * WM;
  constexpr int kAChunks = kBM * (kFK / 16) / kThreads;   // 16-byte chunks per thread: 4
  constexpr int kWChunks = kFBN * (kFK / 16) / kThreads;  // 8 / WM
  using Stage = FStage<WM>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Stage* st = reinterpret_cast<Stage*>(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.y * kBM;
  const int n0 = blockIdx.x * kFBN;
  const int toks = min(kBM, m - t0);
  const int rows = min(kFBN, n - n0);
  const rsrc_t ra = make_rsrc(a + static_cast<size_t>(t0) * k, static_cast<uint32_t>(toks) * static_cast<uint32_t>(k));
  const rsrc_t rw = make_rsrc(w + static_cast<size_t>(n0) * k, static_cast<uint32_t>(rows) * static_cast<uint32_t>(k));
  // chunk c = tid + kThreads i: row c / kFCh, 16-byte column c % kFCh (the
  // column is the same for every i since kThreads is a multiple of kFCh)
  constexpr int kFCh = kFK / 16;  // 16-byte chunks per staged row
  const int scol = 16 * (tid % kFCh);
  const int srow0 = tid / kFCh;
  constexpr int kRowStep = kThreads / kFCh;
  // two register sets of staging loads: the loads of stage s + 3 are issued
  // while stage s + 1 waits in the other set for its LDS store, so every
  // load has two stages of compute to arrive (one set held one stage, short
  // of the L2 / HBM latency at these rates)
  uint4 la0[kAChunks], lw0[kWChunks], la1[kAChunks], lw1[kWChunks];
  auto load = [&](int s, uint4 (&la)[kAChunks], uint4 (&lw)[kWChunks]) {
    const int col = s * kFK + scol;
    const bool in = col < k;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
      la[i] = buf_load16(ra, in ? static_cast<uint32_t>(srow0 + kRowStep * i) * k + col : kOob);
#pragma unroll
    for (int i = 0; i < kWChunks; ++i)
      lw[i] = buf_load16(rw, in ? static_cast<uint32_t>(srow0 + kRowStep * i) * k + col : kOob);
  };
  auto store = [&](Stage& S, const uint4 (&la)[kAChunks], const uint4 (&lw)[kWChunks]) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
      *reinterpret_cast<uint4*>(&S.a[(srow0 + kRowStep * i) * kFStride + scol]) = la[i];
#pragma unroll
    for (int i = 0; i < kWChunks; ++i)
      *reinterpret_cast<uint4*>(&S.w[(srow0 + kRowStep * i) * kFStride + scol]) = lw[i];
  };
  v16f acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int wt = 0; wt < 2; ++wt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ti][wt][i] = 0.f;
  const int r32 = lane & 31, kh = lane >> 5;
  auto compute = [&](const Stage& S) {
#pragma unroll
    for (int ks = 0; ks < kFK / 64; ++ks) {
      const int kb = ks * 64 + 32 * kh;
      v8i av[2], bv[2];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) av[ti] = *reinterpret_cast<const v8i*>(&S.a[(wm * 64 + ti * 32 + r32) * kFStride + kb]);
#pragma unroll
      for (int wt = 0; wt < 2; ++wt) bv[wt] = *reinterpret_cast<const v8i*>(&S.w[(wn * 64 + wt * 32 + r32) * kFStride + kb]);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int wt = 0; wt < 2; ++wt)
          acc[ti][wt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[ti], bv[wt], acc[ti][wt], 0, 0, 0, 0, 0, 0);
    }
  };
  // Stage s is in LDS buffer s & 1; stage s + 1 waits in one register set,
  // stage s + 2 is in flight in the other.  No load is conditional: stages
  // past k read zeros (an odd stage count runs one stage of zeros, which adds
  // exact zeros), so the compiler can count the loads in flight.
  const int nst = (k + kFK - 1) / kFK;
  load(0, la0, lw0);
  store(st[0], la0, lw0);
  load(1, la1, lw1);
  load(2, la0, lw0);
  __syncthreads();
  for (int s = 0; s < nst; s += 2) {
    compute(st[0]);
    // stage s + 1 to the buffer stage s - 1 used (every wavefront left it at
    // the previous barrier), then the loads of stage s + 3
    store(st[1], la1, lw1);
    load(s + 3, la1, lw1);
    __syncthreads();
    compute(st[1]);
    store(st[0], la0, lw0);
    load(s + 4, la0, lw0);
    __syncthreads();
  }
  // epilogue: D rounded to bfloat16 (nearest even) and widened, times the
  // token's absmax/448, then times the weight row's absmax/448
#pragma unroll
  for (int wt = 0; wt < 2; ++wt) {
    const int r = wn * 64 + wt * 32 + r32;
    if (r >= rows) continue;
    const float wa = w_absmax[n0 + r];
    const float f2 = (wa == 0.f ? 1.f : wa) / kE4m3Max;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = wm * 64 + ti * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
        if (t < toks) {
          const float aa = a_absmax[t0 + t];
          const float f1 = (aa == 0.f ? 1.f : aa) / kE4m3Max;
          const float db = __uint_as_float(float_to_bf16_rne(acc[ti][wt][i]) << 16);
          y[static_cast<size_t>(t0 + t) * n + n0 + r] = (db * f1) * f2;
        }
      }
    }
  }
}

template <int WM>
hipError_t launch_gemm_wm(const uint8_t* a, const float* a_absmax, const uint8_t* w, const float* w_absmax, float* y,
                          int m, int n, int k, hipStream_t stream) {
  const size_t lds = 2 * sizeof(FStage<WM>);
  const hipError_t e = lds_opt_in(reinterpret_cast<const void*>(fp8_gemm_kernel<WM>), lds);
  if (e != hipSuccess) return e;
  const dim3 grid((n + kFBN - 1) / kFBN, (m + 64 * WM - 1) / (64 * WM));
  fp8_gemm_kernel<WM><<<grid, dim3(128 * WM), lds, stream>>>(a, a_absmax, w, w_absmax, y, m, n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_absmax_rows(const float* x, int rows, int cols, float* absmax, hipStream_t stream) {
  const bool vec = cols % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
  if (vec)
    absmax_rows_kernel<true><<<dim3(rows), dim3(256), 0, stream>>>(x, cols, absmax);
  else
    absmax_rows_kernel<false><<<dim3(rows), dim3(256), 0, stream>>>(x, cols, absmax);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_rows(const float* x, int rows, int cols, const float* absmax, uint8_t* q,
                                    hipStream_t stream) {
  const bool vec = cols % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0;
  const size_t units = static_cast<size_t>(rows) * static_cast<size_t>(cols) / (vec ? 16 : 1);
  const size_t blocks = (units + 255) / 256;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  if (vec)
    quantize_rows_kernel<true><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(x, absmax, cols, units, q);
  else
    quantize_rows_kernel<false><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(x, absmax, cols, units, q);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t* a, const float* a_absmax, const uint8_t* w, const float* w_absmax,
                           float* y, int m, int n, int k, hipStream_t stream) {
  // 128 x 128 tiles (four wavefronts, 74 KiB of LDS: two workgroups per
  // compute unit).  256 x 128 tiles with eight wavefronts were slower or equal
  // on every prefill shape (107 / 273 / 108 / 284 us against 98 / 270 / 108 /
  // 245 us for gate/up and down at 512 / 2048 tokens), as were 64-byte k stages.
  return launch_gemm_wm<2>(a, a_absmax, w, w_absmax, y, m, n, k, stream);
}

}  // namespace q4k
