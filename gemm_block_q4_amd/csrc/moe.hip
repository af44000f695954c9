// Top-k MoE: routing for the grouped prefill pass and the combine step, gfx950.
//
// "libmir-cuda 0.1.0 -- .../nvfp4/selected/micro_moe.rs",
// DirectNvFp4MoeBf16::new / execute: per token a list of selected expert ids
// and a routing weight per selection; one group per (token, selection) pair.
// The routing kernel sorts the pairs by expert and cuts each expert's run
// into row tiles for the grouped MMQ passes.  The expert passes of the FFN
// write one output row per (token, slot) pair; the combine kernel adds the
// top_k weighted pair rows of every token in slot order (deterministic),
// skipping pairs whose id is outside [0, n_experts).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

// y[t][c] = sum over the valid slots s of wts[t][s] * y_pair[t * top_k + s][c],
// in slot order.  VEC: four consecutive columns per thread (16-byte loads and
// stores; hidden % 4 == 0 and 16-byte aligned rows), else one.
template <bool VEC>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y_pair,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ ids,
                                                          int m, int top_k, int n_experts,
                                                          int hidden, float* __restrict__ y) {
  constexpr int V = VEC ? 4 : 1;
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * V;
  if (t >= m || c >= hidden) return;
  // eight slots per round: all their loads are issued (on clamped, valid
  // indices) before the first is used; the sum stays in slot order
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < top_k; s0 += 8) {
    bool ok[8];
    float w[8], v[8][V];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t * top_k + min(s0 + i, top_k - 1);
      const int id = ids[p];
      ok[i] = s0 + i < top_k && id >= 0 && id < n_experts;
      w[i] = wts[p];
      const float* src = y_pair + static_cast<size_t>(p) * hidden + c;
      if constexpr (VEC) {
        const float4 q = *reinterpret_cast<const float4*>(src);
        v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
      } else {
        v[i][0] = *src;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] = ok[i] ? fmaf(w[i], v[i][j], acc[j]) : acc[j];
  }
  float* dst = y + static_cast<size_t>(t) * hidden + c;
  if constexpr (VEC) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    *dst = acc[0];
  }
}

// One workgroup: per-expert pair counts by LDS atomics, an exclusive scan of
// the counts and of the tile counts over the experts (wavefront 0: a run of
// experts per lane, then a lane scan), the tile table, then every valid pair
// placed at its expert's next list position.
__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t* __restrict__ ids, int pairs,
                                                         int n_experts, int tile_rows,
                                                         int32_t* __restrict__ list,
                                                         int4* __restrict__ tiles,
                                                         int32_t* __restrict__ count) {
  extern __shared__ int route_lds[];
  int* cnt = route_lds;
  int* cur = route_lds + n_experts;
  const int tid = threadIdx.x;
  for (int e = tid; e < n_experts; e += 1024) cnt[e] = 0;
  __syncthreads();
  // eight ids per thread in flight at a time (one load round per 8192 pairs)
  for (int p0 = 0; p0 < pairs; p0 += 8 * 1024) {
    int e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + tid + 1024 * i;
      e[i] = p < pairs ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e[i] >= 0 && e[i] < n_experts) atomicAdd(&cnt[e[i]], 1);
  }
  __syncthreads();
  if (tid < 64) {
    const int per = (n_experts + 63) / 64;
    const int lo = min(n_experts, tid * per), hi = min(n_experts, lo + per);
    int rows = 0, ntiles = 0;
    for (int e = lo; e < hi; ++e) {
      rows += cnt[e];
      ntiles += (cnt[e] + tile_rows - 1) / tile_rows;
    }
    int rs = rows, ts = ntiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int r = __shfl_up(rs, off, 64), t = __shfl_up(ts, off, 64);
      if (tid >= off) {
        rs += r;
        ts += t;
      }
    }
    int row = rs - rows, tile = ts - ntiles;
    for (int e = lo; e < hi; ++e) {
      const int c = cnt[e];
      cur[e] = row;
      for (int j = 0; j * tile_rows < c; ++j) tiles[tile++] = make_int4(e, row + j * tile_rows, min(tile_rows, c - j * tile_rows), 0);
      row += c;
    }
    if (tid == 63) count[0] = ts;
  }
  __syncthreads();
  for (int p0 = 0; p0 < pairs; p0 += 8 * 1024) {
    int e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = p0 + tid + 1024 * i;
      e[i] = p < pairs ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e[i] >= 0 && e[i] < n_experts) list[atomicAdd(&cur[e[i]], 1)] = p0 + tid + 1024 * i;
  }
}

}  // namespace

hipError_t launch_moe_combine(const float* y_pair, const float* wts, const int32_t* ids, int m,
                              int top_k, int n_experts, int hidden, float* y,
                              hipStream_t stream) {
  const bool vec = hidden % 4 == 0 && reinterpret_cast<uintptr_t>(y_pair) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(y) % 16 == 0;
  if (vec) {
    const dim3 grid((hidden / 4 + 255) / 256, m);
    moe_combine_kernel<true><<<grid, dim3(256), 0, stream>>>(y_pair, wts, ids, m, top_k, n_experts, hidden, y);
  } else {
    const dim3 grid((hidden + 255) / 256, m);
    moe_combine_kernel<false><<<grid, dim3(256), 0, stream>>>(y_pair, wts, ids, m, top_k, n_experts, hidden, y);
  }
  return hipGetLastError();
}

hipError_t launch_moe_route(const int32_t* ids, int pairs, int n_experts, int tile_rows, int32_t* list,
                            int32_t* tiles, int32_t* count, hipStream_t stream) {
  if (n_experts < 1 || n_experts > kMoeRouteMaxExperts || pairs < 1 || tile_rows < 1) return hipErrorInvalidValue;
  const size_t lds = 2 * sizeof(int) * static_cast<size_t>(n_experts);
  moe_route_kernel<<<dim3(1), dim3(1024), lds, stream>>>(ids, pairs, n_experts, tile_rows, list,
                                                         reinterpret_cast<int4*>(tiles), count);
  return hipGetLastError();
}

}  // namespace q4k
