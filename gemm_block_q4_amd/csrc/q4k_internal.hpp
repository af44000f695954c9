// Host-side launchers shared between the C ABI layer and the kernel files.
// All launchers assume validated arguments and return the HIP error of the
// launch (hipSuccess when nothing went wrong).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4k {

// Lets `kern` use `lds` bytes of dynamic LDS on the current device: above the
// default 64 KiB limit the kernel is opted in (hipFuncSetAttribute) once per
// (kernel, device) pair; the registry of done pairs is guarded by a mutex, so
// concurrent callers on any devices are safe.
hipError_t lds_opt_in(const void* kern, size_t lds);

// GEMV over one dense matrix, or one of the two MoE passes over expert banks
// (expert e's matrix at e * mat_bytes).
struct GemvArgs {
  const uint8_t* w;      // weight bank (expert 0 at offset 0)
  const uint8_t* w_up;   // up bank for the fused gate/up pass, else nullptr
  size_t mat_bytes;      // bytes per expert matrix
  const void* x;         // activations, row stride ldx elements
  int x_bf16;            // 1: x holds bf16 values, 0: f32
  int ldx;
  float* y;              // output, row stride ldy
  int ldy;
  int n;                 // output rows per matrix
  int k;                 // input columns (multiple of 256)
  int m;                 // tokens (rows of x / y in the dense mode)
  // MoE (ids == nullptr: one dense matrix).  Pair p = t * top_k + s routes
  // token t to expert ids[p]; grid row p runs the rows of that expert on x
  // row p / top_k (x_by_token) or p and writes y row p.  Ids outside
  // [0, n_experts) are skipped.
  const int32_t* ids;
  const float* wts;  // routing weights (the fused down pass)
  int x_by_token;
  int top_k;
  int n_experts;
  int pairs;
  // Split k (matrix-core kernel, one dense f32 matrix, 2..8 tokens):
  // splits == 2 runs every row group as two workgroups over the two halves of
  // the blocks, each adding its sums to y with atomic adds; y must be zero on
  // entry.  0 + a + b rounds the same in either order, so the result does not
  // depend on which half lands first.  splits <= 1: no split.
  int splits;
  // f32 values this launch sets to zero (for a later split launch), or nullptr
  float* zero_out;
  int zero_n;
};

// Splits (1 or 2) the matrix-core kernel takes for m tokens on an [n][k]
// matrix when the caller has zeroed y.
int gemv_mfma_splits(int m, int n, int k);

// Dispatches to the VALU kernel (few tokens) or the matrix-core kernel.
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_valu(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t stream);
// MoE down projection on h rows (x = h [pairs][k], x_by_token = 0) with the
// slot-order combine folded in: writes y[t] for every token.  Needs rows that
// fit one wavefront (k <= 4096); hipErrorNotSupported otherwise.
hipError_t launch_moe_down(const GemvArgs& a, hipStream_t stream);

// Load-time Q4_K quantiser: x [rows][cols] (f32 or bf16) -> block_q4_K.
hipError_t launch_quantize_q4k(const void* x, int x_bf16, int rows, int cols, uint8_t* w,
                               hipStream_t stream);

hipError_t launch_q8_1_quantize(const void* x, int x_bf16, int m, int k, int8_t* qs,
                                uint32_t* ds, hipStream_t stream);

struct MmqArgs {
  const uint8_t* w;      // gate (or single) weights [n][k/256]
  const uint8_t* w_up;   // up weights for the fused SwiGLU pass, else nullptr
  const int8_t* qs;      // Q8_1 quants [m][k]
  const uint32_t* ds;    // Q8_1 scale/sum words [m][k/32]
  float* y;              // [m][n] f32 (h = silu(g) * u when w_up is set)
  // single-matrix pass without k split: when set, y is not written and the
  // result goes here as bfloat16 (rounded to nearest even) instead
  uint16_t* y_bf16;
  // fused gate/up pass only (n % 64 == 0): h is quantised to Q8_1 in the
  // epilogue into q_out [m][n] and d_out [m][n/32] instead of stored to y
  int8_t* q_out;
  uint32_t* d_out;
  int32_t* partials;     // test hook: [m][n][k/32] int32 instead of y
  int m, n, k;
  // k split of the single-matrix pass (splits > 1): split z covers k blocks
  // [z * split_blocks, (z + 1) * split_blocks) and writes its partial sum to
  // y + z * split_stride; mmq_split_reduce adds the planes.  splits <= 1:
  // one pass over all of k into y.
  int splits, split_blocks;
  size_t split_stride;
  // Grouped (MoE prefill) pass when group_tiles is set: grid row g below
  // *group_count runs tile g = {expert e, first row r0, rows, 0} of a row
  // space sorted by expert; e's matrices sit at e * group_mat_bytes of w and
  // w_up.  Row r of the tile reads qs/ds row group_list[r] / group_top_k
  // (group_top_k > 0: the pairs' token rows) or row r (group_top_k == 0);
  // q_out/d_out rows are r, y rows are group_list[r] (group_scatter) or r.
  // group_grid_rows grid rows are launched; the rest exit at once.  No k
  // split, no partials.
  const int32_t* group_tiles;
  const int32_t* group_count;
  const int32_t* group_list;
  size_t group_mat_bytes;
  int group_top_k;
  int group_scatter;
  int group_grid_rows;
  // Dense passes over part of the rows: row tiles [row_tile0, row_tile0 +
  // row_tiles) of the workgroup's row count (64 per matrix in the fused
  // gate/up pass); row_tiles 0: all rows.
  int row_tile0, row_tiles;
  // Fused gate/up pass with a k split (splits > 1, split_blocks as above):
  // split z writes its gate and up sums (before silu * mul) to the planes
  // gu_parts [z][2][m][row_tiles * 64], rows counted from row_tile0 * 64;
  // launch_mmq_gu_finish adds them in split order and writes Q8_1(h).
  float* gu_parts;
};

hipError_t launch_mmq(const MmqArgs& a, hipStream_t stream);

// Q8_1(silu(g) * u) of rows [row0, row0 + rows) of an [m][n] h from the
// planes of a k-split fused gate/up pass (parts [splits][2][m][rows]), the
// splits added in order; the quantisation arithmetic of the fused epilogue.
// rows and row0 are multiples of 32.
hipError_t launch_mmq_gu_finish(const float* parts, int splits, int m, int rows, int row0, int n,
                                int8_t* q_out, uint32_t* d_out, hipStream_t stream);

// Q8_1-activation decode GEMV: y [m][n] = reference dot of Q8_1 rows with the
// Q4_K rows, 1 <= m <= 8, 256 <= k <= 32768 (validated by the caller).
hipError_t launch_q8_gemv(const uint8_t* w, const int8_t* qs, const uint32_t* ds, float* y, int m,
                          int n, int k, hipStream_t stream);
// Q6_K GEMV, one f32 token: y [n] = dequant(w) [n][k] . x, 256 <= k <= 32768.
hipError_t launch_q6k_gemv(const uint8_t* w, const float* x, float* y, int n, int k, hipStream_t stream);

// Gate/up form: h [m][n] = silu(gate . x) * (up . x), both matrices [n][k].
hipError_t launch_q8_gemv_gu(const uint8_t* w_gate, const uint8_t* w_up, const int8_t* qs,
                             const uint32_t* ds, float* h, int m, int n, int k, hipStream_t stream);

// Number of k splits (1 .. max_splits) for the single-matrix MMQ pass of an
// m x n x k product on a device with `cus` compute units: the one that
// minimises the busiest compute unit's share of k blocks (a workgroup fills a
// compute unit), fewer splits on ties.
int mmq_choose_splits(int m, int n, int k, int max_splits, int cus);

// y[i] = sum_{z < splits} parts[z * stride + i] in order z = 0, 1, ...
// (count and stride multiples of 4, 16-byte aligned planes).
hipError_t launch_mmq_split_reduce(const float* parts, int splits, size_t stride, size_t count,
                                   float* y, hipStream_t stream);

// Plain read of `bytes` (a multiple of 16, 16-byte aligned) from `buf`, one
// 16-byte load per thread; `sink` is written only for a fixed bit pattern.
hipError_t launch_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// MoE routing for the grouped prefill pass: list [pairs] = the pair indices
// with a valid id, sorted by expert (order within an expert unspecified);
// tiles [max_tiles][4] = {expert, first list position, rows (<= tile_rows),
// 0} covering each expert's positions in order; count[0] = number of tiles.
// n_experts <= kMoeRouteMaxExperts; max_tiles >= moe_route_max_tiles(...).
constexpr int kMoeRouteMaxExperts = 4096;
inline int moe_route_max_tiles(int pairs, int n_experts, int tile_rows) {
  return pairs / tile_rows + (n_experts < pairs ? n_experts : pairs) + 1;
}
hipError_t launch_moe_route(const int32_t* ids, int pairs, int n_experts, int tile_rows, int32_t* list,
                            int32_t* tiles, int32_t* count, hipStream_t stream);

// y[t] = sum_{s < top_k} wts[t][s] * y_pair[t * top_k + s] in slot order
// (pairs with an id outside [0, n_experts) skipped).
hipError_t launch_moe_combine(const float* y_pair, const float* wts, const int32_t* ids, int m,
                              int top_k, int n_experts, int hidden, float* y, hipStream_t stream);


// Per-row FP8 (E4M3) recipe.  absmax [rows] = max |x| of each f32 row;
// q [rows][cols] = E4M3 codes of x * 448/absmax (16-byte paths when the
// shapes and pointers allow, else one value per thread); y [m][n] =
// bf16(A_fp8 . W_fp8^T) * (a/448) * (w/448) for k % 16 == 0 and k <= 2^20.
hipError_t launch_fp8_absmax_rows(const float* x, int rows, int cols, float* absmax, hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const float* x, int rows, int cols, const float* absmax, uint8_t* q,
                                    hipStream_t stream);
hipError_t launch_fp8_gemm(const uint8_t* a, const float* a_absmax, const uint8_t* w, const float* w_absmax,
                           float* y, int m, int n, int k, hipStream_t stream);

}  // namespace q4k
