"""Plain CPU oracle for the Q4_K SwiGLU feed-forward hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gemm_block_q4_amd/csrc``) and imports nothing from it.

Everything here is deliberately slow and literal: numpy in float64 unless a
step is defined in a narrower type (the Q8_1 encoding is defined in binary32
and binary16 and is reproduced bit for bit).  A library matmul is used as the
one primitive for dense dot products; there is no blocking or fusion.

Sources (the pages), cited by title and item:

* "realizar 0.8.5 -- src/cuda/executor/layers/ffn.rs": ``fused_ffn_swiglu_gpu``
  (the FFN is down(swiglu(gate(x), up(x))), a SwiGLU of a gate and an up
  projection feeding a down projection) and ``fused_ffn_swiglu_gpu_true_dp4a``
  (activations quantised to Q8_1, a per-block scale plus 32 int8 values, with
  the scales applied after the integer dot).
* "realizar 0.8.5 -- src/cuda/executor/q4k_gemv_cached_uses.rs":
  ``q4k_gemv_cached`` (Q4_K GEMV, f32 input of length k, f32 output of length
  n, k a multiple of 256).
* "spark_model/layers/ops/q4k_mmq.rs" (atlas docs): constants ``QK_K`` and
  ``Q4K_BLOCK_BYTES`` (256 weights per 144-byte block_q4_K),
  ``q4k_weight_bytes``, ``quantize_weight_q4k`` (names the GGML block_q4_K
  format), ``quantize_act_q8_1`` and ``q4k_mmq_gemm`` (C[m,n] = A_q8[m,k] x
  W_q4k[n,k]^T) and the file header (prefill pipeline: activations to Q8_1,
  then the MMQ, for gate/up and for down).
* "libmir-cuda 0.1.0 -- .../nvfp4/selected/micro_moe.rs":
  ``DirectNvFp4MoeBf16::execute`` (small-batch top-k MoE: per token a list of
  selected experts and a routing weight per selection) and ``validate`` (gate
  and up banks equal, down bank transposed).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* The byte layout of block_q4_K is GGML's published one: fp16 ``d`` at bytes
  0-1, fp16 ``dmin`` at 2-3, twelve bytes of packed 6-bit (scale, min) pairs
  at 4-15, 128 bytes of 4-bit quants at 16-143.  A weight is
  ``d*sc_j*q - dmin*m_j`` for its 32-weight sub-block j.
* Q8_1: per 32 values, ``d = amax/127`` in binary32, ``q = round-half-even(x/d)``
  in binary32, the scale stored as binary16 (round to nearest even,
  saturating at 65504 when the rounding would overflow, in which case the
  block is quantised with 65504) and the block sum stored as the exact
  integer ``S = sum(q)`` (int16).  A binary16
  block sum ``fp16(d*S)`` overflows for the prefill intermediate activations
  of the synthetic workload, so the integer is kept instead.
* The MMQ result is the reference dot
  ``y[t,n] = sum_j (d*sc_j)[n] * d16[t,j] * P[t,n,j] - (dmin*m_j)[n] * d16[t,j] * S[t,j]``
  with ``P`` the exact int32 dot of the 32 quants of sub-block j.

Parity pins for every function live in ``tests/test_oracle_*.py``.  The one
point left "parity unpinned": bit compatibility with block_q4_K files written
by GGML itself (no such file or printed test vector exists on the pages).
"""

from __future__ import annotations

import numpy as np

# -- block format -------------------------------------------------------------

#: Weights per Q4_K super-block ("q4k_mmq.rs", const ``QK_K``).
QK_K = 256
#: Bytes per block_q4_K ("q4k_mmq.rs", const ``Q4K_BLOCK_BYTES``).
Q4K_BLOCK_BYTES = 144
#: Weights per sub-block, each with its own 6-bit scale and min (GGML layout).
SUB_BLOCK = 32
#: Values per Q8_1 activation block ("ffn.rs", doc of the DP4A FFN: a
#: per-block scale and 32 int8 values).
Q8_1_BLOCK = 32
#: Largest finite binary16 value and the smallest binary32 value that rounds
#: (to nearest even) past it to infinity.
F16_MAX = 65504.0
F16_OVERFLOW = 65520.0


def q4k_weight_bytes(rows: int, cols: int) -> int:
    """Bytes of a Q4_K matrix [rows, cols] ("q4k_mmq.rs", ``q4k_weight_bytes``).

    ``cols`` must be a multiple of 256 (the page's precondition; the GEMV
    launcher in "q4k_gemv_cached_uses.rs" requires k divisible by 256 too).
    """
    if rows < 0 or cols < 0 or cols % QK_K:
        raise ValueError("cols must be a non-negative multiple of 256")
    return rows * (cols // QK_K) * Q4K_BLOCK_BYTES


def _blocks(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """View raw Q4_K bytes as uint8 [rows, cols/256, 144] (row-major blocks)."""
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if w.size != q4k_weight_bytes(rows, cols):
        raise ValueError("weight buffer size does not match rows x cols")
    return w.reshape(rows, cols // QK_K, Q4K_BLOCK_BYTES)


def f16_bits_to_f64(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """Little-endian byte pair -> IEEE binary16 value, widened exactly to f64."""
    bits = lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float64)


def unpack_scale_min(scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Twelve packed bytes -> eight 6-bit scales and eight 6-bit mins.

    GGML block_q4_K layout: sub-blocks 0-3 keep their scale in the low six
    bits of byte j and their min in the low six bits of byte j+4; sub-blocks
    4-7 take the low four bits from byte j+4 (scale: low nibble, min: high
    nibble) and the high two bits from the top two bits of byte j-4 (scale)
    and byte j (min).
    """
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    mn = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        mn[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 0x0F) | ((s[..., j - 4] >> 6) << 4)
        mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, mn


def pack_scale_min(sc: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """Inverse of :func:`unpack_scale_min` (eight 6-bit pairs -> 12 bytes)."""
    sc = np.asarray(sc, dtype=np.int64)
    mn = np.asarray(mn, dtype=np.int64)
    if sc.min(initial=0) < 0 or sc.max(initial=0) > 63 or mn.min(initial=0) < 0 or mn.max(initial=0) > 63:
        raise ValueError("scales and mins are 6-bit")
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.int64)
    for j in range(4):
        out[..., j] = (sc[..., j] & 63) | ((sc[..., j + 4] >> 4) << 6)
        out[..., j + 4] = (mn[..., j] & 63) | ((mn[..., j + 4] >> 4) << 6)
        out[..., j + 8] = (sc[..., j + 4] & 0x0F) | ((mn[..., j + 4] & 0x0F) << 4)
    return out.astype(np.uint8)


def unpack_quants(qs: np.ndarray) -> np.ndarray:
    """128 packed bytes -> 256 quants 0..15 in weight order.

    GGML block_q4_K layout: for g = 0..3 and l = 0..31, weight 64g+l is the
    low nibble of byte 32g+l (sub-block 2g) and weight 64g+32+l is the high
    nibble of the same byte (sub-block 2g+1).
    """
    qs = np.asarray(qs, dtype=np.uint8)
    q = np.empty(qs.shape[:-1] + (QK_K,), dtype=np.uint8)
    for g in range(4):
        chunk = qs[..., 32 * g: 32 * g + 32]
        q[..., 64 * g: 64 * g + 32] = chunk & 0x0F
        q[..., 64 * g + 32: 64 * g + 64] = chunk >> 4
    return q


def block_fields(w: np.ndarray, rows: int, cols: int):
    """Decode every block of a Q4_K matrix into its fields.

    Returns ``d, dmin`` (f64 [rows, nb]), ``sc, mn`` (int [rows, nb, 8]) and
    ``q`` (uint8 [rows, nb, 256]) with ``nb = cols/256``.
    """
    b = _blocks(w, rows, cols)
    d = f16_bits_to_f64(b[..., 0], b[..., 1])
    dmin = f16_bits_to_f64(b[..., 2], b[..., 3])
    sc, mn = unpack_scale_min(b[..., 4:16])
    q = unpack_quants(b[..., 16:144])
    return d, dmin, sc, mn, q


def dequantize(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q4_K matrix -> f64 [rows, cols]; each weight is ``d*sc_j*q - dmin*m_j``.

    For the synthetic weights (d, dmin in [1e-3, 1e-2]) every value is exact
    in f64: the two products need at most 21 and 17 significant bits and
    their exponents differ by a few binades only.
    """
    d, dmin, sc, mn, q = block_fields(w, rows, cols)
    nb = cols // QK_K
    qf = q.reshape(rows, nb, 8, SUB_BLOCK).astype(np.float64)
    scale = (d[..., None] * sc)[..., None]          # d * sc_j
    minv = (dmin[..., None] * mn)[..., None]        # dmin * m_j
    return (scale * qf - minv).reshape(rows, cols)


# -- decode: dequant-fused GEMV (f32 activations) ----------------------------

def gemv(w: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_k w[n, k] * x[t, k] in f64 ("q4k_gemv_cached_uses.rs").

    ``x`` is f32 [m, cols] (exact in f64); returns f64 [m, rows].
    """
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != cols:
        raise ValueError("x must be [m, cols]")
    return x.astype(np.float64) @ dequantize(w, rows, cols).T


# -- Q8_1 activation quantisation --------------------------------------------

def pack_quants(q: np.ndarray) -> np.ndarray:
    """Inverse of :func:`unpack_quants` (256 quants 0..15 -> 128 bytes)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.max(initial=0) > 15:
        raise ValueError("quants are 4-bit")
    out = np.empty(q.shape[:-1] + (128,), dtype=np.uint8)
    for g in range(4):
        out[..., 32 * g: 32 * g + 32] = q[..., 64 * g: 64 * g + 32] | (q[..., 64 * g + 32: 64 * g + 64] << 4)
    return out


def _f16_saturating(v: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 (nearest even), 65504 where the rounding would overflow."""
    v = np.asarray(v, dtype=np.float32)
    return np.where(v >= F16_OVERFLOW, np.float32(F16_MAX), v).astype(np.float16)


def q4k_quantize(x: np.ndarray) -> np.ndarray:
    """block_q4_K encoding of weights [rows, cols], cols a multiple of 256.

    "q4k_mmq.rs", ``quantize_weight_q4k``, names a load-time quantiser to the
    GGML block_q4_K format but prints no algorithm.  Reading taken (the
    plainest fit of the format, not GGML's scale search), every step in
    binary32 with round-to-nearest-even, per 32-value sub-block j of a
    256-value block:

    * ``lo_j = min(0, min w)``, ``hi_j = max w``; the offset ``o_j = 0 - lo_j``
      (+0, not -0, when nothing is negative) and the step
      ``s_j = (hi_j - lo_j) / 15`` (+0 when ``hi_j == lo_j``, so that zeros
      of either sign give the same bytes) map the sub-block onto 0..15;
    * ``d = binary16(max_j s_j / 63)``, ``dmin = binary16(max_j o_j / 63)``
      (saturating at 65504 as for Q8_1);
    * ``sc_j = rint(s_j / d)`` and ``m_j = rint(o_j / dmin)``, clamped to
      0..63 (0 when the divisor is 0);
    * ``q = rint((w + dmin*m_j) / (d*sc_j))`` clamped to 0..15 (0 when
      ``d*sc_j`` is 0), so ``d*sc_j*q - dmin*m_j`` is the nearest value on
      the block's grid.

    bf16 input is widened to f32 exactly by the caller.  Returns uint8
    [rows * cols/256 * 144].  Input must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % QK_K:
        raise ValueError("x must be [rows, cols] with cols a multiple of 256")
    if not np.all(np.isfinite(x)):
        raise ValueError("Q4_K input must be finite")
    rows, cols = x.shape
    nb = cols // QK_K
    xb = x.reshape(rows, nb, 8, SUB_BLOCK)
    lo = np.minimum(xb.min(axis=-1), np.float32(0.0))
    hi = xb.max(axis=-1)
    o = (np.float32(0.0) - lo).astype(np.float32)  # +0 when nothing is negative
    s = np.where(hi > lo, (hi - lo).astype(np.float32) / np.float32(15.0), np.float32(0.0)).astype(np.float32)
    d16 = _f16_saturating(s.max(axis=-1) / np.float32(63.0))
    m16 = _f16_saturating(o.max(axis=-1) / np.float32(63.0))
    d = d16.astype(np.float32)[..., None]
    dmin = m16.astype(np.float32)[..., None]
    sc = np.where(d > 0, np.clip(np.rint(s / np.where(d > 0, d, np.float32(1.0))), 0, 63), 0).astype(np.int64)
    mn = np.where(dmin > 0, np.clip(np.rint(o / np.where(dmin > 0, dmin, np.float32(1.0))), 0, 63), 0).astype(np.int64)
    ds = (d * sc.astype(np.float32)).astype(np.float32)          # exact: 11 x 6 bits
    dm = (dmin * mn.astype(np.float32)).astype(np.float32)
    num = (xb + dm[..., None]).astype(np.float32)
    ratio = (num / np.where(ds > 0, ds, np.float32(1.0))[..., None]).astype(np.float32)
    q = np.where(ds[..., None] > 0, np.clip(np.rint(ratio), 0, 15), 0).astype(np.uint8)
    out = np.empty((rows, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(rows, nb, 2)
    out[..., 2:4] = m16.view(np.uint8).reshape(rows, nb, 2)
    out[..., 4:16] = pack_scale_min(sc, mn)
    out[..., 16:] = pack_quants(q.reshape(rows, nb, QK_K))
    return out.reshape(-1)


def q8_1_quantize(x: np.ndarray):
    """Q8_1 encoding of f32 activations [m, k], k a multiple of 32.

    Per 32-value block ("ffn.rs", DP4A FFN doc: per-block scale + 32 int8;
    "q4k_mmq.rs", ``quantize_act_q8_1``):

    * ``amax = max |x_i|`` (exact);
    * if ``amax == 0`` every quant is 0 and the scale is +0;
    * else ``d = amax / 127`` in binary32, ``q_i = rint(x_i / d)`` with the
      division in binary32 and rounding half to even (clamped to +-127, a
      guard that never fires);
    * stored: ``d16 = binary16(d)`` (round to nearest even, subnormals kept)
      and the exact block sum ``S = sum q_i``;
    * if ``binary16(d)`` would overflow (``d >= 65520``), the scale saturates:
      ``d = 65504`` is stored and used as the divisor, so values beyond
      127 * 65504 clamp to +-127 (the pages leave scale overflow open).

    Returns ``qs`` int8 [m, k], ``d16`` float16 [m, k/32], ``S`` int16
    [m, k/32].  Input must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % Q8_1_BLOCK:
        raise ValueError("x must be [m, k] with k a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("Q8_1 input must be finite")
    m, k = x.shape
    xb = x.reshape(m, k // Q8_1_BLOCK, Q8_1_BLOCK)
    amax = np.max(np.abs(xb), axis=-1)                       # float32, exact
    d = amax / np.float32(127.0)                             # binary32 RNE
    # a scale whose binary16 rounding would overflow saturates at 65504 and
    # the block is quantised with that stored scale instead
    sat = d >= F16_OVERFLOW
    d = np.where(sat, np.float32(F16_MAX), d).astype(np.float32)
    safe = np.where(amax > 0, d, np.float32(1.0)).astype(np.float32)
    ratio = (xb / safe[..., None]).astype(np.float32)        # binary32 RNE
    q = np.clip(np.rint(ratio), -127, 127)                   # half to even
    q = np.where(amax[..., None] > 0, q, 0).astype(np.int8)
    d16 = np.where(amax > 0, d, np.float32(0.0)).astype(np.float16)
    s = q.astype(np.int32).sum(axis=-1).astype(np.int16)
    return q.reshape(m, k), d16, s


def q8_1_dequantize(qs: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """The activation the integer GEMM sees: ``x_hat = d16 * q`` (f64)."""
    m, k = qs.shape
    return (np.asarray(d16, dtype=np.float64)[..., None]
            * qs.reshape(m, k // Q8_1_BLOCK, Q8_1_BLOCK).astype(np.float64)).reshape(m, k)


def pack_ds(d16: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Planar per-block word: bits 0-15 = d16, bits 16-31 = S (two's complement)."""
    lo = np.asarray(d16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    hi = np.asarray(s, dtype=np.int16).view(np.uint16).astype(np.uint32)
    return lo | (hi << 16)


def unpack_ds(ds: np.ndarray):
    """Inverse of :func:`pack_ds`."""
    ds = np.asarray(ds, dtype=np.uint32)
    d16 = (ds & 0xFFFF).astype(np.uint16).view(np.float16)
    s = (ds >> 16).astype(np.uint16).view(np.int16)
    return d16, s


# -- prefill: Q8_1 x Q4_K reference dot (MMQ) ---------------------------------

def mmq_partials_token(w: np.ndarray, rows: int, cols: int, qs_t: np.ndarray,
                       fields=None) -> np.ndarray:
    """Integer partials of one token: P[n, j] = sum_{i<32} q_w[n, 32j+i] * q_a[32j+i].

    ``qs_t`` is int8 [cols].  Returns int64 [rows, cols/32] (every value fits
    int32: |P| <= 32 * 15 * 127).
    """
    if fields is None:
        fields = block_fields(w, rows, cols)
    # |q_w * q_a| <= 15 * 127 fits int16 and a 32-term sum fits int32, so the
    # narrow integer types below are exact
    q = fields[4].reshape(rows, cols).astype(np.int16)
    prod = q * np.asarray(qs_t, dtype=np.int16)[None, :]
    return prod.reshape(rows, cols // SUB_BLOCK, SUB_BLOCK).sum(axis=-1, dtype=np.int64)


def mmq_partials(w: np.ndarray, rows: int, cols: int, qs: np.ndarray) -> np.ndarray:
    """P[t, n, j] for every token (small shapes only): int64 [m, rows, cols/32]."""
    fields = block_fields(w, rows, cols)
    return np.stack([mmq_partials_token(w, rows, cols, qs[t], fields)
                     for t in range(qs.shape[0])])


def mmq(w: np.ndarray, rows: int, cols: int, qs: np.ndarray, d16: np.ndarray,
        s: np.ndarray, tokens=None) -> np.ndarray:
    """Reference dot of Q8_1 activations with a Q4_K matrix, f64 [len(tokens), rows].

    y[t, n] = sum over sub-blocks j of
        (d * sc_j)[n] * d16[t, j] * P[t, n, j]  -  (dmin * m_j)[n] * d16[t, j] * S[t, j]

    ("q4k_mmq.rs", ``q4k_mmq_gemm``: C = A_q8 x W_q4k^T; "ffn.rs", DP4A FFN
    doc: integer dot first, scales applied at the end).  With the integer
    block sum this equals sum_k w_hat[n, k] * x_hat[t, k] exactly in real
    arithmetic.  ``tokens`` selects rows of the activation (default: all).
    """
    d, dmin, sc, mn, _ = fields = block_fields(w, rows, cols)
    nsub = cols // SUB_BLOCK
    sw = (d[..., None] * sc).reshape(rows, nsub)            # d * sc_j, exact
    mw = (dmin[..., None] * mn).reshape(rows, nsub)         # dmin * m_j, exact
    da = np.asarray(d16, dtype=np.float64)
    sa = np.asarray(s, dtype=np.float64)
    if tokens is None:
        tokens = range(qs.shape[0])
    out = []
    for t in tokens:
        p = mmq_partials_token(w, rows, cols, qs[t], fields).astype(np.float64)
        out.append(((sw * p) * da[t][None, :] - (mw * (da[t] * sa[t])[None, :])).sum(axis=1))
    return np.array(out, dtype=np.float64).reshape(len(out), rows)


# -- SwiGLU and the FFN --------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in f64 (-> -0 as g -> -inf)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u ("ffn.rs", ``fused_ffn_swiglu_gpu`` step 3)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def ffn_decode(w_gate, w_up, w_down, hidden: int, inter: int, x: np.ndarray) -> np.ndarray:
    """Decode FFN, y = down(silu(gate(x)) * up(x)), f32 activations, all in f64.

    "ffn.rs", ``fused_ffn_swiglu_gpu``: gate GEMV, up GEMV, SwiGLU, down GEMV;
    no activation is quantised.  ``x`` f32 [m, hidden] -> f64 [m, hidden].
    """
    g = gemv(w_gate, inter, hidden, x)
    u = gemv(w_up, inter, hidden, x)
    h = swiglu(g, u)
    return h @ dequantize(w_down, hidden, inter).T


def ffn_prefill(w_gate, w_up, w_down, hidden: int, inter: int, x: np.ndarray,
                tokens=None) -> np.ndarray:
    """Prefill FFN at the same quantisation points as the integer path.

    "q4k_mmq.rs" header: activations -> Q8_1, MMQ for gate and up; SwiGLU;
    the activated vector -> Q8_1, MMQ for down ("ffn.rs", DP4A FFN, steps
    1-6).  ``x`` is the f32 widening of the bf16 input.  The gate/up results
    and the SwiGLU are f64; ``h`` is rounded to f32 before its quantisation
    (the Q8_1 encoding is defined on binary32 input).  Every step is per
    token, so ``tokens`` may select a subset; returns f64 [len, hidden].
    The DP4A decode FFN of "ffn.rs" (``fused_ffn_swiglu_gpu_true_dp4a``)
    computes the same steps for a few tokens, so this is its oracle too.
    """
    x = np.asarray(x, dtype=np.float32)
    if tokens is None:
        tokens = list(range(x.shape[0]))
    xs = x[list(tokens)]
    qx, dx, sx = q8_1_quantize(xs)
    g = mmq(w_gate, inter, hidden, qx, dx, sx)
    u = mmq(w_up, inter, hidden, qx, dx, sx)
    h = swiglu(g, u).astype(np.float32)
    qh, dh, sh = q8_1_quantize(h)
    return mmq(w_down, hidden, inter, qh, dh, sh)


def moe_decode(bank_gate, bank_up, bank_down, n_experts: int, hidden: int, inter: int,
               x: np.ndarray, ids: np.ndarray, wts: np.ndarray) -> np.ndarray:
    """Small-batch top-k MoE FFN (f32 activations, f64 arithmetic).

    "micro_moe.rs", ``DirectNvFp4MoeBf16::execute``: per token a list of
    selected experts and one routing weight per selection.  Expert e's
    gate/up matrices are [inter, hidden] and its down matrix is
    [hidden, inter] (``validate``: down is the transposed shape), each at
    offset e * q4k_weight_bytes(rows, cols) of its bank.
    y[t] = sum over slots s, in slot order, of wts[t, s] * FFN_{ids[t, s]}(x[t]).
    """
    gu_bytes = q4k_weight_bytes(inter, hidden)
    dn_bytes = q4k_weight_bytes(hidden, inter)
    bank_gate = np.asarray(bank_gate, dtype=np.uint8).reshape(-1)
    bank_up = np.asarray(bank_up, dtype=np.uint8).reshape(-1)
    bank_down = np.asarray(bank_down, dtype=np.uint8).reshape(-1)
    x = np.asarray(x, dtype=np.float32)
    m, top_k = ids.shape
    y = np.zeros((m, hidden), dtype=np.float64)
    for t in range(m):
        for s in range(top_k):
            e = int(ids[t, s])
            if not 0 <= e < n_experts:
                raise ValueError("expert id out of range")
            wg = bank_gate[e * gu_bytes:(e + 1) * gu_bytes]
            wu = bank_up[e * gu_bytes:(e + 1) * gu_bytes]
            wd = bank_down[e * dn_bytes:(e + 1) * dn_bytes]
            y[t] += float(wts[t, s]) * ffn_decode(wg, wu, wd, hidden, inter, x[t:t + 1])[0]
    return y


def moe_prefill(bank_gate, bank_up, bank_down, n_experts: int, hidden: int, inter: int,
                x: np.ndarray, ids: np.ndarray, wts: np.ndarray, tokens=None) -> np.ndarray:
    """Top-k MoE FFN for many tokens at the prefill quantisation points.

    "micro_moe.rs", ``DirectNvFp4MoeBf16::new`` / ``execute``: one group per
    (token, selected expert) pair, each pair's FFN run on its expert's
    matrices, combined per token with the routing weights.  Each pair's FFN
    is the prefill FFN of ``ffn_prefill`` ("q4k_mmq.rs" pipeline: Q8_1(x),
    MMQ gate and up, SwiGLU, h to f32 and Q8_1, MMQ down); every step is per
    token, so a pair's result depends only on x[t] and its expert.
    y[t] = sum over slots s, in slot order, of wts[t, s] * FFN_{ids[t, s]}(x[t]);
    ``tokens`` selects the returned rows.  Returns f64 [len, hidden].
    """
    gu_bytes = q4k_weight_bytes(inter, hidden)
    dn_bytes = q4k_weight_bytes(hidden, inter)
    bank_gate = np.asarray(bank_gate, dtype=np.uint8).reshape(-1)
    bank_up = np.asarray(bank_up, dtype=np.uint8).reshape(-1)
    bank_down = np.asarray(bank_down, dtype=np.uint8).reshape(-1)
    x = np.asarray(x, dtype=np.float32)
    m, top_k = ids.shape
    if tokens is None:
        tokens = list(range(m))
    y = np.zeros((len(tokens), hidden), dtype=np.float64)
    for i, t in enumerate(tokens):
        for s in range(top_k):
            e = int(ids[t, s])
            if not 0 <= e < n_experts:
                raise ValueError("expert id out of range")
            wg = bank_gate[e * gu_bytes:(e + 1) * gu_bytes]
            wu = bank_up[e * gu_bytes:(e + 1) * gu_bytes]
            wd = bank_down[e * dn_bytes:(e + 1) * dn_bytes]
            y[i] += float(wts[t, s]) * ffn_prefill(wg, wu, wd, hidden, inter, x[t:t + 1])[0]
    return y


# -- acceptance metrics (used by the parity tests) -----------------------------

def row_norms(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """||w_hat_n||_2 for every row (f64)."""
    return np.sqrt((dequantize(w, rows, cols) ** 2).sum(axis=1))


def normalized_max_error(y: np.ndarray, y_ref: np.ndarray, w_norms: np.ndarray,
                         x_norms: np.ndarray) -> float:
    """max_{t,n} |y - y_ref| / (||w_n|| * ||x_t||); a zero denominator needs y == 0."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.asarray(x_norms, dtype=np.float64)[:, None] * np.asarray(w_norms, dtype=np.float64)[None, :]
    err = np.abs(y - y_ref)
    zero = den == 0
    if np.any(err[zero] != 0):
        return float("inf")
    den = np.where(zero, 1.0, den)
    return float((err / den).max(initial=0.0))


def relative_l2(y: np.ndarray, y_ref: np.ndarray) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over every element."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
