"""Independent pure-Python decoders used to pin the oracle on tiny inputs.

Written from the block_q4_K description (GGML layout: fp16 d, fp16 dmin,
twelve bytes of 6-bit scale/min fields, 128 bytes of nibbles) as a walk over
bit positions, with no numpy and no code shared with ``oracle/``.
"""

from __future__ import annotations

import math
import struct


def bits_of(data: bytes) -> list[int]:
    """Little-endian bit string: bit 8*i + b is bit b of byte i."""
    return [(data[i] >> b) & 1 for i in range(len(data)) for b in range(8)]


def field(bits: list[int], start: int, width: int) -> int:
    return sum(bits[start + i] << i for i in range(width))


def scale_min_bitwalk(scales12: bytes) -> tuple[list[int], list[int]]:
    """(sc_j, m_j) for j = 0..7 read straight off bit positions.

    j < 4: sc = bits [8j, 8j+6), m = bits [8(j+4), 8(j+4)+6).
    j >= 4: sc = bits [8(j+4), +4) | bits [8(j-4)+6, +2) << 4,
            m  = bits [8(j+4)+4, +4) | bits [8j+6, +2) << 4.
    """
    b = bits_of(scales12)
    sc, mn = [], []
    for j in range(8):
        if j < 4:
            sc.append(field(b, 8 * j, 6))
            mn.append(field(b, 8 * (j + 4), 6))
        else:
            sc.append(field(b, 8 * (j + 4), 4) | (field(b, 8 * (j - 4) + 6, 2) << 4))
            mn.append(field(b, 8 * (j + 4) + 4, 4) | (field(b, 8 * j + 6, 2) << 4))
    return sc, mn


def quant_bitwalk(qs128: bytes, i: int) -> int:
    """Quant of weight i (0..255): byte 32*(i//64) + (i%64)%32, low nibble if
    (i%64) < 32 else high nibble."""
    g, r = divmod(i, 64)
    byte = qs128[32 * g + (r % 32)]
    return byte & 15 if r < 32 else byte >> 4


def half(data: bytes) -> float:
    return struct.unpack("<e", data)[0]


def decode_block(block: bytes) -> list[float]:
    """All 256 weights of one 144-byte block as Python floats (double)."""
    assert len(block) == 144
    d = half(block[0:2])
    dmin = half(block[2:4])
    sc, mn = scale_min_bitwalk(block[4:16])
    out = []
    for i in range(256):
        j = i // 32
        out.append(d * sc[j] * quant_bitwalk(block[16:144], i) - dmin * mn[j])
    return out


def decode_matrix(w: bytes, rows: int, cols: int) -> list[list[float]]:
    nb = cols // 256
    mat = []
    for r in range(rows):
        row = []
        for b in range(nb):
            off = (r * nb + b) * 144
            row.extend(decode_block(w[off:off + 144]))
        mat.append(row)
    return mat


def f32(v: float) -> float:
    """Round a double to binary32 (nearest even) and back."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f16(v: float) -> float:
    """Round a double to binary16 (nearest even, subnormals kept)."""
    return struct.unpack("<e", struct.pack("<e", v))[0]


def rint_even(v: float) -> int:
    """Round half to even."""
    fl = math.floor(v)
    diff = v - fl
    if diff > 0.5:
        return fl + 1
    if diff < 0.5:
        return fl
    return fl if fl % 2 == 0 else fl + 1


def q8_1_block(xs: list[float]) -> tuple[list[int], float, int]:
    """One 32-value Q8_1 block from binary32 inputs: (quants, d16, sum).

    The binary32 quotient is formed in double and rounded once to binary32,
    which is the correctly rounded binary32 quotient of binary32 operands.
    """
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return [0] * len(xs), 0.0, 0
    d = f32(amax / 127.0)
    if d >= 65520.0:          # binary16 would overflow: saturate the scale
        d = 65504.0
    q = [max(-127, min(127, rint_even(f32(v / d)))) for v in xs]
    return q, f16(d), sum(q)
