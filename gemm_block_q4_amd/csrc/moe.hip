// Small-batch top-k MoE: routing table and deterministic combine, gfx950.
//
// "libmir-cuda 0.1.0 -- .../nvfp4/selected/micro_moe.rs",
// DirectNvFp4MoeBf16::execute: per token a list of selected expert ids and a
// routing weight per selection; groups = tokens * selected.  The pairs
// (t, s) are grouped by expert so that each selected expert's weights are
// streamed once for all of its tokens: the route kernel assigns every
// distinct expert (ascending id) one or more slots of at most `cap` pairs,
// the GEMV kernels run one grid row per slot, and the combine kernel adds the
// top_k weighted pair outputs of every token in slot order.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

// One workgroup; pairs <= 64 * 64 is guaranteed by the host (m <= 8).
__global__ __launch_bounds__(64) void moe_route_kernel(const int32_t* __restrict__ ids, int pairs,
                                                      int top_k, int n_experts, int cap,
                                                      SlotTable tab, int slots) {
  __shared__ int sid[64 * 8];
  __shared__ int sfirst[64 * 8];
  __shared__ int schunks[64 * 8];
  const int tid = threadIdx.x;
  for (int p = tid; p < pairs; p += 64) {
    const int e = ids[p];
    sid[p] = (e >= 0 && e < n_experts) ? e : -1;
  }
  __syncthreads();
  // For every pair: is it the first pair of its expert, and how many pairs
  // share the expert.
  for (int p = tid; p < pairs; p += 64) {
    const int e = sid[p];
    int first = e >= 0 ? 1 : 0, count = 0;
    for (int q = 0; q < pairs; ++q) {
      if (sid[q] == e) {
        ++count;
        if (q < p) first = 0;
      }
    }
    sfirst[p] = first;
    schunks[p] = first ? (count + cap - 1) / cap : 0;
  }
  __syncthreads();
  for (int s = tid; s < slots; s += 64) {
    tab.expert[s] = -1;
    tab.count[s] = 0;
  }
  __syncthreads();
  for (int p = tid; p < pairs; p += 64) {
    const int e = sid[p];
    if (e < 0) continue;
    // Slot base of expert e: chunks of every distinct expert with a smaller id.
    int base = 0, pos = 0, count = 0;
    for (int q = 0; q < pairs; ++q) {
      if (sfirst[q] && sid[q] < e) base += schunks[q];
      if (sid[q] == e) {
        if (q < p) ++pos;
        ++count;
      }
    }
    const int slot = base + pos / cap;
    const int within = pos % cap;
    if (slot < slots) {
      if (within == 0) {
        tab.expert[slot] = e;
        tab.count[slot] = min(cap, count - (pos / cap) * cap);
      }
      tab.xrow[slot * kMaxTokens + within] = p / top_k;
      tab.yrow[slot * kMaxTokens + within] = p;
    }
  }
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y_pair,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ ids,
                                                          int m, int top_k, int n_experts,
                                                          int hidden, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (t >= m || c >= hidden) return;
  float acc = 0.f;
  for (int s = 0; s < top_k; ++s) {
    const int p = t * top_k + s;
    const int e = ids[p];
    if (e < 0 || e >= n_experts) continue;
    acc = fmaf(wts[p], y_pair[static_cast<size_t>(p) * hidden + c], acc);
  }
  y[static_cast<size_t>(t) * hidden + c] = acc;
}

}  // namespace

hipError_t launch_moe_route(const int32_t* ids, int m, int top_k, int n_experts,
                            const SlotTable& t, int slots, hipStream_t stream) {
  const int cap = m < kMaxTokens ? m : kMaxTokens;
  moe_route_kernel<<<dim3(1), dim3(64), 0, stream>>>(ids, m * top_k, top_k, n_experts, cap, t,
                                                    slots);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* y_pair, const float* wts, const int32_t* ids, int m,
                              int top_k, int n_experts, int hidden, float* y,
                              hipStream_t stream) {
  const dim3 grid((hidden + 255) / 256, m);
  moe_combine_kernel<<<grid, dim3(256), 0, stream>>>(y_pair, wts, ids, m, top_k, n_experts,
                                                     hidden, y);
  return hipGetLastError();
}

}  // namespace q4k
