/*
 * q4k.h -- C ABI of the MI355X (gfx950) Q4_K SwiGLU feed-forward library.
 *
 * The library computes the feed-forward block y = down(silu(gate(x)) * up(x))
 * with weights stored as GGML-style block_q4_K, in two regimes: a
 * dequant-fused GEMV for a few tokens (decode) and a Q8_1-activation x Q4_K
 * integer GEMM (MMQ) for many tokens (prefill).  Sources, by page title:
 *   - "realizar 0.8.5 -- src/cuda/executor/layers/ffn.rs": fused_ffn_swiglu_gpu
 *     (the FFN), fused_ffn_swiglu_gpu_true_dp4a (Q8_1 activations, per-block
 *     scale + 32 int8, scales applied after the integer dot).
 *   - "realizar 0.8.5 -- src/cuda/executor/q4k_gemv_cached_uses.rs":
 *     q4k_gemv_cached / _async (Q4_K GEMV, f32 x of length k, f32 y of length
 *     n, k divisible by 256) and q4k_gemv_indexed_async (a null weight pointer
 *     is rejected before any launch).
 *   - "spark_model/layers/ops/q4k_mmq.rs": QK_K = 256, Q4K_BLOCK_BYTES = 144,
 *     q4k_weight_bytes, quantize_act_q8_1, q4k_mmq_gemm (C = A_q8 x W_q4k^T),
 *     and the prefill pipeline in the file header.
 *   - "libmir-cuda 0.1.0 -- .../nvfp4/selected/micro_moe.rs":
 *     DirectNvFp4MoeBf16::execute (top-k MoE: selected expert ids and a
 *     routing weight per selection) and validate / elements (bank shapes,
 *     overflow-checked sizes).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; the caller owns every buffer and keeps it alive until
 *     the stream has run the call.  The library allocates nothing and keeps no
 *     data between calls (the per-device caches below aside).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call is
 *     asynchronous on it; nothing synchronises inside the library.
 *   - Arguments are validated on the host before any launch; on error nothing
 *     is launched and a q4k_status code is returned.  Q4K_ERR_LAUNCH reports
 *     a failure returned by the HIP runtime after a launch.
 *   - Weight matrices, activations, quantised activations and the workspace
 *     must be 16-byte aligned (a 144-byte block is nine 16-byte words, so all
 *     blocks stay aligned).  Routing ids and weights need 4-byte alignment.
 *   - Calls are reentrant and may come from several host threads at once.
 *     The only process-wide state is a cache per device ordinal (whether it is
 *     a gfx950, its compute-unit count: atomics) and the set of (kernel,
 *     device) pairs already opted into more than 64 KiB of LDS (guarded by a
 *     mutex); each is written once per device and never changes a result.
 *
 * block_q4_K (GGML layout): bytes 0-1 fp16 d, 2-3 fp16 dmin, 4-15 twelve
 * bytes of packed 6-bit (scale, min) pairs for eight 32-weight sub-blocks,
 * 16-143 the 256 4-bit quants (weight 64g+l is the low nibble of byte 32g+l,
 * weight 64g+32+l its high nibble).  Weight value: d*sc_j*q - dmin*m_j.
 * A Q4_K matrix [rows][cols] stores row r's blocks at
 * r*(cols/256) ... r*(cols/256) + cols/256 - 1 (row-major).
 *
 * Q8_1 (planar layout of this library): qs int8 [m][k] row-major and ds
 * uint32 [m][k/32], where bits 0-15 hold the binary16 scale d and bits 16-31
 * hold the block sum S = sum of the 32 quants as int16 (two's complement).
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weights per super-block and bytes per block_q4_K ("q4k_mmq.rs", QK_K and
   Q4K_BLOCK_BYTES). */
#define Q4K_QK 256
#define Q4K_BLOCK_BYTES 144
/* Values per Q8_1 activation block ("ffn.rs", DP4A FFN doc). */
#define Q4K_Q8_1_BLOCK 32
/* Most tokens the decode regime (dequant-fused GEMV) takes per call. */
#define Q4K_DECODE_MAX_TOKENS 8
/* Bytes of the fixed scratch buffer behind ffn_swiglu_q4k_noalloc (64 MiB
   per device). */
#define Q4K_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

typedef enum {
  Q4K_OK = 0,
  Q4K_ERR_NULL = 1,      /* a required pointer is NULL */
  Q4K_ERR_SHAPE = 2,     /* a size is out of range or not a required multiple */
  Q4K_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  Q4K_ERR_OVERFLOW = 4,  /* a derived size overflows */
  Q4K_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
  Q4K_ERR_LAUNCH = 6,    /* the HIP runtime reported an error for a launch */
  Q4K_ERR_DEVICE = 7,    /* the current device is not gfx950 */
  Q4K_ERR_SCRATCH = 8    /* needs more than Q4K_NOALLOC_SCRATCH_BYTES (ffn_swiglu_q4k_noalloc) */
} q4k_status;

typedef enum { Q4K_F32 = 0, Q4K_BF16 = 1 } q4k_dtype;

typedef enum {
  Q4K_REGIME_AUTO = 0,    /* decode when m <= Q4K_DECODE_MAX_TOKENS, else prefill */
  Q4K_REGIME_DECODE = 1,  /* f32 activations, dequant-fused GEMV */
  Q4K_REGIME_PREFILL = 2, /* Q8_1 activations, integer MMQ */
  Q4K_REGIME_DECODE_Q8 = 3 /* Q8_1 activations, integer-dot GEMV (m <= 8, dense only) */
} q4k_regime;

/* Host.  Bytes of a Q4_K matrix [rows][cols]: rows * (cols/256) * 144
   ("q4k_mmq.rs", q4k_weight_bytes).  Returns 0 when rows < 0, cols < 0,
   cols % 256 != 0 or the size overflows. */
size_t q4k_weight_bytes(int rows, int cols);

/* Host.  Static description of a status code (never NULL). */
const char* q4k_status_string(int status);

/* Decode GEMV ("q4k_gemv_cached_uses.rs", q4k_gemv_cached_async):
     y[t][j] = sum_i dequant(w)[j][i] * x[t][i]   for t < m, j < n.
   w: device, block_q4_K [n][k/256]; x: device f32 [m][k] row-major;
   y: device f32 [m][n] row-major, overwritten.  1 <= m <= 8, n >= 1,
   256 <= k <= 32768, k % 256 == 0.  Weights are never rounded.  For one token
   each 64-value slice of x is held as an integer with 21 significant bits
   relative to the slice maximum (exact integer dot products, f32 scaling and
   accumulation); for 2..8 tokens x is split into two binary16 parts for the
   matrix cores.  Either way max |err| / (||w_j|| ||x_t||) stays far below
   1e-5.  A non-finite x gives non-finite outputs.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q4k_gemv(const void* w, const float* x, float* y, int m, int n, int k, void* stream);

/* Load-time Q4_K weight quantiser ("q4k_mmq.rs", quantize_weight_q4k:
   weights are encoded to GGML block_q4_K at load time; the pages print no
   algorithm).  The plain min/max fit, every step in binary32 with
   round-to-nearest-even, for each 32-value sub-block j of a 256-value block:
     lo = min(0, min x), hi = max x, o = 0 - lo, s = hi > lo ? (hi - lo)/15 : 0
     d = binary16(max_j s / 63), dmin = binary16(max_j o / 63)  (65504 where
     the rounding would overflow)
     sc_j = rint(s_j / d), m_j = rint(o_j / dmin), clamped to 0..63 (0 when
     the divisor is 0)
     q = rint((x + dmin*m_j) / (d*sc_j)), clamped to 0..15 (0 when d*sc_j = 0)
   Bit-exact by construction (IEEE operations only).  x: device [rows][cols]
   of x_dtype (Q4K_F32, or Q4K_BF16 widened exactly), 16-byte aligned;
   w: device block_q4_K [rows][cols/256] (q4k_weight_bytes(rows, cols)
   bytes), 16-byte aligned, overwritten.
   rows >= 1, cols >= 256, cols % 256 == 0.  Inputs must be finite
   (non-finite input gives undefined codes but never faults).
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q4k_quantize(const void* x, int x_dtype, int rows, int cols, void* w, void* stream);

/* Q8_1 activation quantisation ("q4k_mmq.rs", quantize_act_q8_1; "ffn.rs",
   q8_quantize_async): for each row t and 32-value block b of x,
     amax = max |x|, d = amax / 127 (binary32), q = rint(x / d) (binary32
     division, half to even), ds = binary16(d) | (sum q) << 16;
   an all-zero block stores q = 0 and ds = 0; a block with d >= 65520 (whose
   binary16 rounding would overflow) stores d = 65504 and is quantised with
   it, so values beyond 127 * 65504 clamp to +-127.  Bit-exact by construction.
   x: device [m][k] of x_dtype (Q4K_F32 or Q4K_BF16, bf16 widened exactly);
   qs: device int8 [m][k]; ds: device uint32 [m][k/32].  m >= 1, k >= 32,
   k % 32 == 0.  Inputs must be finite (non-finite input gives undefined
   codes but never faults). */
int q8_1_quantize(const void* x, int x_dtype, int m, int k, int8_t* qs, uint32_t* ds,
                  void* stream);

/* Prefill integer GEMM ("q4k_mmq.rs", q4k_mmq_gemm: C[m,n] = A_q8[m,k] x
   W_q4k[n,k]^T; "ffn.rs", DP4A FFN doc: integer dot, then scales):
     P[t][j][b] = sum_{i<32} q_w[j][32b+i] * q_a[t][32b+i]      (int32, exact)
     y[t][j] = sum_b (d*sc)[j][b] * d_a[t][b] * P - (dmin*m)[j][b] * d_a[t][b] * S[t][b]
   w: device block_q4_K [n][k/256]; qs/ds: device Q8_1 of the activations
   [m][k] (as written by q8_1_quantize); y: device f32 [m][n], overwritten.
   1 <= m <= 64 * 65535, n >= 1, 256 <= k <= 2^20, k % 256 == 0.  Integer products are exact
   (int8 MFMA); scales are applied in f32. */
int q4k_mmq(const void* w, const int8_t* qs, const uint32_t* ds, float* y, int m, int n,
            int k, void* stream);

/* The same product with the result stored as bfloat16 from the tile
   epilogue ("q4k_mmq.rs" header: the MMQ writes bf16 itself, no separate
   cast): y[t][j] = bf16 rounding (to nearest even) of the value q4k_mmq
   stores as f32, bit for bit.  y: device uint16 (bfloat16 bits) [m][n],
   2-byte aligned, overwritten.  Same shape rules and errors as q4k_mmq. */
int q4k_mmq_bf16(const void* w, const int8_t* qs, const uint32_t* ds, uint16_t* y, int m, int n,
                 int k, void* stream);

/* Q8_1-activation decode GEMV ("ffn.rs", fused_ffn_swiglu_gpu_true_dp4a:
   Q8_1 activations, integer dot products with the Q4_K quants, scales
   applied afterwards): the q4k_mmq product for a decode step's few tokens,
     P[t][j][b] = sum_{i<32} q_w[j][32b+i] * q_a[t][32b+i]      (int32, exact)
     y[t][j] = sum_b (d*sc)[j][b] * d_a[t][b] * P - (dmin*m)[j][b] * d_a[t][b] * S[t][b]
   with P from 4-byte integer dot products on the vector ALUs (each weight row
   is read once for all m tokens).  w: device block_q4_K [n][k/256]; qs/ds:
   device Q8_1 of the activations [m][k] (as written by q8_1_quantize); y:
   device f32 [m][n], overwritten.  1 <= m <= 8, n >= 1, 256 <= k <= 32768,
   k % 256 == 0; ds must be 8-byte aligned (each lane reads the words of two
   sub-blocks at once).  Scales are applied in f32; the result agrees with
   q4k_mmq to f32 rounding.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q4k_q8_gemv(const void* w, const int8_t* qs, const uint32_t* ds, float* y, int m, int n,
                int k, void* stream);

/* Host.  Bytes of a Q6_K matrix [rows][cols]: rows * (cols/256) * 210
   (GGML's block_q6_K: 128 bytes of low 4 bits, 64 of high 2 bits, 16 int8
   scales, an fp16 d).  Returns 0 when rows < 0, cols < 0, cols % 256 != 0 or
   the size overflows. */
size_t q6k_weight_bytes(int rows, int cols);

/* Q6_K GEMV for the LM head ("q4k_gemv_cached_uses.rs",
   q6k_gemv_cached_async: the Q4_K GEMV for Q6_K weights, one f32 token):
     y[j] = sum_i dequant(w)[j][i] * x[i]   for j < n,
   with weight i of a block = d * scales[i/16] * (u - 32), u its 6-bit value
   (low nibble of ql[64h + 32(r&1) + l] for quarter r < 2 of half h, high
   nibble for r >= 2, high 2 bits = bits 2r..2r+1 of qh[32h + l]).
   w: device, block_q6_K [n][k/256] (210-byte blocks, contiguous rows), 16-byte
   aligned; x: device f32 [k], 16-byte aligned; y: device f32 [n], overwritten.
   n >= 1, 256 <= k <= 32768, k % 256 == 0.  Products and sums in f32.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q6k_gemv(const void* w, const float* x, float* y, int n, int k, void* stream);

/* Test hook on the same device code as q4k_mmq: writes the integer partials
   partials[t][j][b] = P[t][j][b] (int32 [m][n][k/32], device) instead of y.
   Same shape rules as q4k_mmq; meant for small shapes. */
int q4k_test_mmq_partials(const void* w, const int8_t* qs, int m, int n, int k,
                          int32_t* partials, void* stream);

/* Measurement hook: reads `bytes` bytes of device memory at `buf` the
   plainest way (one 16-byte load per thread, 256 threads per workgroup) and
   discards them; `sink` (device, one uint32) is written only if a lane's 16
   bytes XOR to 0x9E3779B9.  Timed beside q4k_gemv on the same weight copies
   it gives the read ceiling the GEMV is compared with; not part of the
   computation.  bytes > 0 and a multiple of 16; buf 16-byte aligned.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q4k_test_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Per-row FP8 (E4M3) prefill recipe ("aprender-serve 0.70.2 --
   src/cuda/executor/layers/cublas_prefill/fp8_recipe.rs", module header,
   fp8_absmax_rows, fp8_quantize_rows, fp8_dequant_outer).  Each activation
   row (token) and each weight row (output channel) has its own scale
   448/absmax; E4M3 is the OCP E4M3FN format (sign, 4 exponent bits with bias
   7, 3 mantissa bits, largest finite value 448, code 0x7F/0xFF NaN, no
   infinity).  A weight is quantised once with fp8_absmax_rows +
   fp8_quantize_rows; per call the activations get the same two steps, then
   fp8_gemm_dequant.

   fp8_absmax_rows: absmax[r] = max_i |x[r][i]| (f32; x finite).
   x: device f32 [rows][cols] row-major; absmax: device f32 [rows],
   overwritten.  rows >= 1, cols >= 1; 4-byte alignment (rows of a multiple of
   4 values at a 16-byte aligned x are read 16 bytes at a time).
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int fp8_absmax_rows(const float* x, int rows, int cols, float* absmax, void* stream);

/* fp8_quantize_rows: q[r][i] = E4M3 code of x[r][i] * s_r, with
   s_r = 448 / absmax[r] as a correctly rounded binary32 quotient (absmax 0
   taken as 1, so s_r = 448) and the binary32 product encoded to the nearest
   E4M3 value, ties to even, magnitudes saturated at 448 (code 0x7E / 0xFE),
   subnormals (multiples of 2^-9 below 2^-6) kept, zeros keeping their sign.
   x: device f32 [rows][cols] row-major, finite (NaN input is not defined);
   absmax: device f32 [rows] (normally fp8_absmax_rows of the same x);
   q: device uint8 [rows][cols], overwritten.  rows >= 1, cols >= 1;
   x and absmax 4-byte aligned (16-byte aligned x and q with cols % 16 == 0
   take the vector path; results do not depend on the path).
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int fp8_quantize_rows(const float* x, int rows, int cols, const float* absmax, uint8_t* q, void* stream);

/* fp8_gemm_dequant: the FP8 GEMM and the outer dequant in one pass,
     D[t][c] = sum_i A[t][i] * W[c][i]   (E4M3 values, f32 accumulation),
     y[t][c] = (bf16(D[t][c]) * (a_absmax[t] / 448)) * (w_absmax[c] / 448),
   where bf16() rounds to bfloat16 (nearest even) as the GEMM's BF16 output
   does, each factor is a correctly rounded binary32 quotient with absmax 0
   taken as 1, and the two products are binary32 in this order.  The products
   of two E4M3 values are exact; only the f32 accumulation order differs from
   an exact sum, by far less than one bfloat16 step of D.
   a: device uint8 [m][k] E4M3 codes (tokens); a_absmax: device f32 [m];
   w: device uint8 [n][k] E4M3 codes (weight rows); w_absmax: device f32 [n];
   y: device f32 [m][n] row-major, overwritten.  1 <= m <= 4194240, n >= 1,
   16 <= k <= 1048576, k % 16 == 0; a and w 16-byte aligned, the rest 4-byte
   aligned.  NaN codes (0x7F, 0xFF) give NaN outputs.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int fp8_gemm_dequant(const uint8_t* a, const float* a_absmax, const uint8_t* w, const float* w_absmax, float* y,
                     int m, int n, int k, void* stream);

/* Host.  Workspace bytes ffn_swiglu_q4k needs for these sizes and regime
   (Q4K_REGIME_AUTO resolves by m as the call does); top_k = 0 for a dense
   FFN.  Returns 0 for invalid sizes. */
size_t ffn_swiglu_q4k_workspace_bytes(int m, int hidden, int inter, int top_k, int regime);

/* SwiGLU feed-forward block ("ffn.rs", fused_ffn_swiglu_gpu and
   fused_ffn_swiglu_gpu_true_dp4a; "q4k_mmq.rs" prefill pipeline;
   "micro_moe.rs" for the MoE form):
     dense (ids == NULL, n_experts == 1):
       y[t] = W_down . (silu(W_gate . x[t]) * (W_up . x[t]))
     MoE (ids != NULL):
       y[t] = sum_{s < top_k} wts[t][s] * FFN_{ids[t][s]}(x[t])   (slot order)
   w_gate, w_up: device banks of n_experts block_q4_K matrices [inter][hidden];
   w_down: device bank of n_experts matrices [hidden][inter]; expert e's matrix
   starts at e * q4k_weight_bytes(rows, cols) in its bank ("micro_moe.rs",
   validate: gate and up equal, down transposed).
   x: device [m][hidden] of x_dtype; y: device f32 [m][hidden], overwritten
   (y may be x itself: every regime reads x completely before y is written).
   ids: device int32 [m][top_k]; wts: device f32 [m][top_k].  An id outside
   [0, n_experts) contributes nothing (device data is not read back).
   Regime: decode = f32 activations through the dequant-fused GEMV (gate and
   up in one pass with silu*mul fused); prefill = x -> Q8_1 -> MMQ gate/up
   with fused silu*mul -> h -> Q8_1 -> MMQ down; decode_q8 ("ffn.rs",
   fused_ffn_swiglu_gpu_true_dp4a) = x -> Q8_1 -> integer-dot gate/up GEMV
   with fused silu*mul -> h (f32) -> Q8_1 -> integer-dot down GEMV, the
   prefill arithmetic for 1 <= m <= 8 tokens (dense only).  MoE in the
   decode regime runs one GEMV pass per (token, slot) pair; MoE in the
   prefill regime ("micro_moe.rs", DirectNvFp4MoeBf16::new: one group per
   pair) sorts the pairs by expert on the device and runs one grouped MMQ
   gate/up pass (token rows gathered, Q8_1(h) written per pair) and one
   grouped MMQ down pass over every (expert, 128-pair tile), then the
   slot-order combine; there n_experts <= 4096, m * hidden <= 2^31 and
   m * top_k * inter <= 2^31.  hidden, inter: multiples of 256 (at most 32768
   in the decode regimes, at most 2^20 in the prefill regime).
   workspace: device, at least ffn_swiglu_q4k_workspace_bytes(...) bytes.
   Errors: Q4K_ERR_NULL, Q4K_ERR_SHAPE, Q4K_ERR_ALIGN, Q4K_ERR_OVERFLOW,
   Q4K_ERR_WORKSPACE, Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int ffn_swiglu_q4k(const void* w_gate, const void* w_up, const void* w_down, int n_experts,
                   const void* x, int x_dtype, int m, int hidden, int inter,
                   const int32_t* ids, const float* wts, int top_k, int regime, float* y,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free form of ffn_swiglu_q4k, for callers that cannot allocate
   device memory or pass a workspace (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc).  Same arguments, results
   and errors as ffn_swiglu_q4k, without workspace / workspace_bytes: the
   intermediate buffers live in a fixed scratch array of
   Q4K_NOALLOC_SCRATCH_BYTES in device memory, one per device, held until the
   process ends.  A call whose layout (ffn_swiglu_q4k_workspace_bytes for the
   same sizes and regime) exceeds it returns Q4K_ERR_SCRATCH and launches
   nothing; e.g. 512 tokens of the 5120/17408 prefill need 48.6 MB.  The call
   itself allocates nothing and calls no allocating routine.  Every call on a
   device shares that device's scratch (no result depends on what a previous
   call left there), so calls that overlap on one device -- on different
   streams, or from different host threads without ordering -- race and must
   not be issued. */
int ffn_swiglu_q4k_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                           int n_experts, const void* x, int x_dtype, int m, int hidden,
                           int inter, const int32_t* ids, const float* wts, int top_k, int regime,
                           float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
