"""Plain CPU oracle for the Q6_K GEMV (the LM head's weight format).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gemm_block_q4_amd/csrc``) and imports nothing from it.

Source (the pages), cited by title and item:

* "realizar 0.8.5 -- src/cuda/executor/q4k_gemv_cached_uses.rs",
  ``q6k_gemv_cached_async``: the Q4_K GEMV's counterpart for Q6_K weights,
  used for the LM head; one f32 input vector of length k, an f32 output of
  length n, k a multiple of 256 for its multi-warp form.

Reading where the page is silent (it names the format only): the byte layout
is GGML's published ``block_q6_K``, 256 weights in 210 bytes:

* bytes 0-127 ``ql``: the low 4 bits of every weight;
* bytes 128-191 ``qh``: the high 2 bits;
* bytes 192-207 ``scales``: 16 signed 8-bit scales, one per 16 weights;
* bytes 208-209 ``d``: binary16 block scale.

Weight i of a block (``h = i // 128`` the half, ``r = (i % 128) // 32`` the
quarter of the half, ``l = i % 32``) takes its low 4 bits from byte
``64h + 32(r % 2) + l`` of ``ql`` (the low nibble for r < 2, the high nibble
for r >= 2) and its high 2 bits from bits ``2r, 2r+1`` of byte ``32h + l`` of
``qh``; with ``u`` that 6-bit value the weight is ``d * scales[i // 16] *
(u - 32)``.

Parity pins: ``tests/test_oracle_q6k.py`` (hand-derived values of a
hand-built block in ``tests/golden/q6k_hand_block.json``, a bit-level decoder
on random blocks, the packing bijection, closed forms, and a pure-Python
GEMV).  Bit compatibility with Q6_K files written by GGML itself is "parity
unpinned": the pages print no such file or test vector.
"""

from __future__ import annotations

import numpy as np

#: Weights per Q6_K super-block (the same 256 as Q4_K).
QK_K = 256
#: Bytes per block_q6_K: 128 + 64 + 16 + 2.
Q6K_BLOCK_BYTES = 210


def q6k_weight_bytes(rows: int, cols: int) -> int:
    """Bytes of a Q6_K matrix [rows, cols]; ``cols`` a multiple of 256."""
    if rows < 0 or cols < 0 or cols % QK_K:
        raise ValueError("cols must be a non-negative multiple of 256")
    return rows * (cols // QK_K) * Q6K_BLOCK_BYTES


def _blocks(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if w.size != q6k_weight_bytes(rows, cols):
        raise ValueError("weight buffer size does not match rows x cols")
    return w.reshape(rows, cols // QK_K, Q6K_BLOCK_BYTES)


def unpack_q6(ql: np.ndarray, qh: np.ndarray) -> np.ndarray:
    """The 256 unsigned 6-bit values (0..63) of blocks [..., 128] and [..., 64]."""
    ql = np.asarray(ql, dtype=np.uint8)
    qh = np.asarray(qh, dtype=np.uint8)
    out = np.empty(ql.shape[:-1] + (QK_K,), dtype=np.uint8)
    for h in range(2):
        for r in range(4):
            lo_bytes = ql[..., 64 * h + 32 * (r % 2): 64 * h + 32 * (r % 2) + 32]
            low = (lo_bytes >> 4) if r >= 2 else (lo_bytes & 0x0F)
            high = (qh[..., 32 * h: 32 * h + 32] >> (2 * r)) & 0x03
            out[..., 128 * h + 32 * r: 128 * h + 32 * r + 32] = low | (high << 4)
    return out


def pack_q6(u: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of :func:`unpack_q6`: 256 values 0..63 -> (ql [128], qh [64])."""
    u = np.asarray(u, dtype=np.uint8)
    if u.max(initial=0) > 63:
        raise ValueError("Q6_K values are 6-bit")
    ql = np.zeros(u.shape[:-1] + (128,), dtype=np.uint8)
    qh = np.zeros(u.shape[:-1] + (64,), dtype=np.uint8)
    for h in range(2):
        for r in range(4):
            v = u[..., 128 * h + 32 * r: 128 * h + 32 * r + 32]
            sl = slice(64 * h + 32 * (r % 2), 64 * h + 32 * (r % 2) + 32)
            ql[..., sl] |= ((v & 0x0F) << 4) if r >= 2 else (v & 0x0F)
            qh[..., 32 * h: 32 * h + 32] |= (v >> 4) << (2 * r)
    return ql, qh


def dequantize(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q6_K bytes -> f64 weights [rows, cols] (``d * scale * (u - 32)``, exact)."""
    b = _blocks(w, rows, cols)
    u = unpack_q6(b[..., 0:128], b[..., 128:192]).astype(np.float64) - 32.0
    sc = b[..., 192:208].view(np.int8).astype(np.float64)
    d = (b[..., 208].astype(np.uint16) | (b[..., 209].astype(np.uint16) << 8)).view(np.float16)
    d = d.astype(np.float64)
    scale = np.repeat(sc, 16, axis=-1) * d[..., None]
    return (scale * u).reshape(rows, cols)


def gemv(w: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_k w[n, k] * x[t, k] in f64 (``q6k_gemv_cached_async``).

    ``x`` is f32 [m, cols]; returns f64 [m, rows].
    """
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != cols:
        raise ValueError("x must be [m, cols]")
    return x.astype(np.float64) @ dequantize(w, rows, cols).T


def row_norms(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Euclidean norm of each dequantised row (f64 [rows])."""
    return np.linalg.norm(dequantize(w, rows, cols), axis=1)
