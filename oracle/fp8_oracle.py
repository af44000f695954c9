"""Plain CPU oracle for the per-row FP8 (E4M3) prefill recipe.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gemm_block_q4_amd/csrc``) and imports nothing from it.

Source (the pages), cited by title and item:

* "aprender-serve 0.70.2 -- src/cuda/executor/layers/cublas_prefill/
  fp8_recipe.rs": the FP8 prefill recipe.  Every activation row (token) and
  every weight row (output channel) gets its own scale; the quantiser keeps
  E4M3 subnormals; the GEMM of the two FP8 matrices writes D in BF16 with
  alpha 1, and the two per-row scales are applied afterwards, in the
  widening of D to f32: ``Y[t, c] = D[t, c] * (a[t]/448) * (w[c]/448)``.
  Items: ``fp8_absmax_rows`` (row max of |x|), ``fp8_quantize_rows`` (x times
  ``448/absmax`` of its row, an all-zero row taking absmax 1, encoded to
  E4M3 with round to nearest even, saturating at 448, subnormals kept),
  ``fp8_dequant_outer`` (BF16 D widened exactly, times ``absmax_t/448``,
  times ``absmax_c/448``, each factor a correctly rounded binary32
  division, zero absmax again taken as 1).

E4M3 here is the OCP "E4M3FN" format the page's encoder targets: sign bit,
4-bit exponent with bias 7, 3-bit mantissa; normal values
``2^(e-7) * (1 + m/8)`` for e in 1..15 (code 0x7F, e = 15 and m = 7, is NaN,
so 448 = ``2^8 * 1.75`` is the largest finite value), subnormals
``m/8 * 2^-6`` for e = 0.

Readings where the page is silent or the PTX is only a sketch (each listed
in the design notes):

* The encoder is the nearest E4M3 value (ties to even) of the binary32
  product ``x * (448/absmax)``, saturated at +-448; the page's bit-level
  steps compute exactly that.  A zero maps to +0 or -0 by its sign.
* D is the exact sum of the products of the two encoded rows (the page's
  cuBLASLt GEMM accumulates in f32; this oracle gives the exact value, the
  GPU's f32 accumulation is checked against it with a stated bound), rounded
  to BF16 (nearest even) as the page's GEMM output is.
* Input must be finite (the page maps NaN to 448 through min.f32; the
  library does not promise that).

Pins: ``tests/test_oracle_fp8.py`` (brute-force nearest-code search over all
256 codes, hand-derived codes, the decode table from the format definition,
saturation and subnormal edges, the GEMM against Python loops).
"""

from __future__ import annotations

import numpy as np

#: Largest finite E4M3 (E4M3FN) value, the page's saturation point.
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN byte codes -> f64 values (0x7F / 0xFF, the NaN codes, give NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0x0F
    m = c & 0x07
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of binary32 values (ties to even), saturating at
    +-448 ("fp8_recipe.rs", fp8_quantize_rows).

    The magnitude is placed on the grid of its binade: for |v| >= 2^-6 the
    step is 2^(E-3) with E the binary exponent of |v|; below 2^-6 the
    subnormal step 2^-9.  Rounding |v| / step to the nearest integer (ties
    to even) gives the significand; a carry into the next binade is a
    larger exponent with mantissa 0."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encoding needs finite input")
    a = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    sign = np.where(np.signbit(v), 0x80, 0x00)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals: q = rne(a * 2^9), 0..8 (8 is the smallest normal's code)
    q = np.rint(a * 512.0).astype(np.int64)
    out = np.where(sub, q, out)
    # normals: a = 2^E * f, 1 <= f < 2; significand on the 3-bit grid
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    E = np.where(np.ldexp(1.0, E + 1) <= a, E + 1, E)
    E = np.where(np.ldexp(1.0, E) > a, E - 1, E)
    f = np.rint(np.ldexp(a, -E) * 8.0).astype(np.int64)  # 8..16, ties to even
    carry = f == 16
    E = np.where(carry, E + 1, E)
    f = np.where(carry, 8, f)
    normal = (E + 7) << 3 | (f - 8)
    out = np.where(sub, out, normal)
    return (out | sign).astype(np.uint8)


def absmax_rows(x: np.ndarray) -> np.ndarray:
    """Row max of |x| ("fp8_recipe.rs", fp8_absmax_rows), f32 [rows]."""
    x = np.asarray(x, dtype=np.float32)
    return np.abs(x).max(axis=1).astype(np.float32)


def row_scale(absmax: np.ndarray) -> np.ndarray:
    """448 / absmax per row as a correctly rounded binary32 quotient; an
    all-zero row takes absmax 1 (scale 448)."""
    am = np.asarray(absmax, dtype=np.float32)
    am = np.where(am == 0, np.float32(1.0), am).astype(np.float32)
    return (np.float32(E4M3_MAX) / am).astype(np.float32)


def quantize_rows(x: np.ndarray, absmax: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """E4M3 codes of x [rows, cols] with one scale per row, and the row absmax.

    Each value is multiplied by its row's ``448/absmax`` in binary32, then
    encoded (``fp8_quantize_rows``)."""
    x = np.asarray(x, dtype=np.float32)
    if absmax is None:
        absmax = absmax_rows(x)
    scale = row_scale(absmax)
    v = (x * scale[:, None]).astype(np.float32)
    return e4m3_encode(v), np.asarray(absmax, dtype=np.float32)


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round f64 values to binary32 and then to bfloat16 (nearest even each
    time), returned as f64: the exact D passes through the f32 value a
    binary32 accumulator would hold before the BF16 store."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def dequant_outer(D: np.ndarray, a_absmax: np.ndarray, w_absmax: np.ndarray) -> np.ndarray:
    """``fp8_dequant_outer``: Y [m, n] from the GEMM result D [m, n] (f64
    values, rounded here to binary32 and then BF16 as the GEMM's BF16 output
    is), widened, times ``a[t]/448`` then times ``w[c]/448`` in binary32
    (each factor a binary32 quotient, zero absmax taken as 1)."""
    Db = bf16_rne(D).astype(np.float32)
    am = np.asarray(a_absmax, dtype=np.float32)
    wm = np.asarray(w_absmax, dtype=np.float32)
    f1 = (np.where(am == 0, np.float32(1.0), am).astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    f2 = (np.where(wm == 0, np.float32(1.0), wm).astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    y = (Db * f1[:, None]).astype(np.float32)
    return (y * f2[None, :]).astype(np.float32)


def gemm_codes(a_codes: np.ndarray, w_codes: np.ndarray) -> np.ndarray:
    """D = A_fp8 . W_fp8^T as the exact sum of the decoded products (f64).

    Every product of two E4M3 values is a multiple of 2^-18 below 2^18, so the
    sums stay exact in f64 while |D| < 2^35."""
    return e4m3_decode(a_codes) @ e4m3_decode(w_codes).T


def gemm_rows(a_codes: np.ndarray, a_absmax: np.ndarray, w_codes: np.ndarray,
              w_absmax: np.ndarray) -> np.ndarray:
    """Y [m, n] of the recipe: the exact D of the two code matrices, then
    ``dequant_outer``."""
    return dequant_outer(gemm_codes(a_codes, w_codes), a_absmax, w_absmax)


def gemm_rows_exact(a_codes, a_absmax, w_codes, w_absmax) -> np.ndarray:
    """The same product without the BF16 rounding of D, in f64 (the value the
    BF16 store approximates)."""
    A = e4m3_decode(a_codes)
    W = e4m3_decode(w_codes)
    am = np.where(np.asarray(a_absmax) == 0, 1.0, np.asarray(a_absmax, dtype=np.float64))
    wm = np.where(np.asarray(w_absmax) == 0, 1.0, np.asarray(w_absmax, dtype=np.float64))
    return (A @ W.T) * (am / E4M3_MAX)[:, None] * (wm / E4M3_MAX)[None, :]
