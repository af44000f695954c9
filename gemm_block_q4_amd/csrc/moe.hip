// Small-batch top-k MoE: the combine step, gfx950.
//
// "libmir-cuda 0.1.0 -- .../nvfp4/selected/micro_moe.rs",
// DirectNvFp4MoeBf16::execute: per token a list of selected expert ids and a
// routing weight per selection.  The expert passes of the FFN write one
// output row per (token, slot) pair; this kernel adds the top_k weighted
// pair rows of every token in slot order (deterministic), skipping pairs
// whose id is outside [0, n_experts).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y_pair,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ ids,
                                                          int m, int top_k, int n_experts,
                                                          int hidden, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (t >= m || c >= hidden) return;
  // eight slots per round: all their loads are issued (on clamped, valid
  // indices) before the first is used; the sum stays in slot order
  float acc = 0.f;
  for (int s0 = 0; s0 < top_k; s0 += 8) {
    int e[8];
    float w[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t * top_k + min(s0 + i, top_k - 1);
      const int id = ids[p];
      e[i] = s0 + i < top_k ? id : -1;
      w[i] = wts[p];
      v[i] = y_pair[static_cast<size_t>(p) * hidden + c];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = e[i] >= 0 && e[i] < n_experts ? fmaf(w[i], v[i], acc) : acc;
  }
  y[static_cast<size_t>(t) * hidden + c] = acc;
}

}  // namespace

hipError_t launch_moe_combine(const float* y_pair, const float* wts, const int32_t* ids, int m,
                              int top_k, int n_experts, int hidden, float* y,
                              hipStream_t stream) {
  const dim3 grid((hidden + 255) / 256, m);
  moe_combine_kernel<<<grid, dim3(256), 0, stream>>>(y_pair, wts, ids, m, top_k, n_experts,
                                                     hidden, y);
  return hipGetLastError();
}

}  // namespace q4k
