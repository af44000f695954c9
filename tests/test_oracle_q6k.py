"""Pins of the Q6_K oracle: hand-derived values, a bit-level decoder, the
packing bijection, closed forms and a pure-Python GEMV."""
import json
import os
import struct

import numpy as np

from gemm_block_q4_amd import synth
from oracle import q6k_oracle as q6

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def hand_block():
    with open(os.path.join(GOLDEN, "q6k_hand_block.json")) as f:
        h = json.load(f)
    block = np.zeros(210, dtype=np.uint8)
    block[0:128] = np.arange(128, dtype=np.uint8)
    block[128:192] = h["qh_byte"]
    block[192:208] = np.array(h["scales"], dtype=np.int8).view(np.uint8)
    block[208:210] = np.array([h["d_bits"]], dtype=np.uint16).view(np.uint8)
    return h, block


def test_hand_block():
    h, block = hand_block()
    w = q6.dequantize(block, 1, 256)[0]
    for pos, val in h["weights"].items():
        assert w[int(pos)] == val, pos


def bitwalk_weight(block: bytes, i: int) -> float:
    """Weight i of one 210-byte block, read bit by bit from the layout."""
    h, r, l = i >> 7, (i >> 5) & 3, i & 31
    low = (block[64 * h + 32 * (r & 1) + l] >> (4 * (r >> 1))) & 15
    high = (block[128 + 32 * h + l] >> (2 * r)) & 3
    sc = struct.unpack("<b", block[192 + i // 16: 193 + i // 16])[0]
    d = struct.unpack("<e", block[208:210])[0]
    return d * sc * ((low | (high << 4)) - 32)


def test_dequant_against_bitwalk_decoder():
    g = synth.rng(20, 1)
    for rows, cols in ((1, 256), (3, 512), (2, 768)):
        w = synth.random_q6k(g, rows, cols)
        raw = bytes(w)
        ref = np.empty((rows, cols))
        nb = cols // 256
        for r in range(rows):
            for c in range(cols):
                b = r * nb + c // 256
                ref[r, c] = bitwalk_weight(raw[210 * b: 210 * b + 210], c % 256)
        assert np.array_equal(q6.dequantize(w, rows, cols), ref)


def test_packing_is_a_bijection():
    g = synth.rng(21, 1)
    u = g.integers(0, 64, (50, 256), dtype=np.uint8)
    ql, qh = q6.pack_q6(u)
    assert np.array_equal(q6.unpack_q6(ql, qh), u)
    # each of the 256 x 6 value bits lands on its own one of the 192 x 8 field bits
    seen = set()
    for i in range(256):
        for bit in range(6):
            one = np.zeros(256, dtype=np.uint8)
            one[i] = 1 << bit
            ql, qh = q6.pack_q6(one)
            field = np.concatenate([ql, qh])
            (pos,) = np.nonzero(field)
            assert len(pos) == 1 and bin(int(field[pos[0]])).count("1") == 1
            seen.add((int(pos[0]), int(field[pos[0]]).bit_length() - 1))
    assert len(seen) == 256 * 6 == 192 * 8


def test_closed_forms():
    # u = 32 everywhere: every weight is zero whatever the scales
    ql, qh = q6.pack_q6(np.full(256, 32, dtype=np.uint8))
    block = np.zeros(210, dtype=np.uint8)
    block[:128], block[128:192] = ql, qh
    block[192:208] = np.arange(16, dtype=np.uint8) * 17
    block[208:210] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)  # d = 1
    assert np.all(q6.dequantize(block, 1, 256) == 0)
    # u = 0 with scale -128 and d = 1: the largest magnitude, +4096
    block[:192] = 0
    block[192:208] = np.array([-128] * 16, dtype=np.int8).view(np.uint8)
    assert np.all(q6.dequantize(block, 1, 256) == 4096.0)
    # u = 63, scale 127, d = 2: 2 * 127 * 31
    ql, qh = q6.pack_q6(np.full(256, 63, dtype=np.uint8))
    block[:128], block[128:192] = ql, qh
    block[192:208] = 127
    block[208:210] = np.array([0x4000], dtype=np.uint16).view(np.uint8)
    assert np.all(q6.dequantize(block, 1, 256) == 2 * 127 * 31)
    # d = 0: zero
    block[208:210] = 0
    assert np.all(q6.dequantize(block, 1, 256) == 0)


def test_gemv_against_python_loops():
    g = synth.rng(22, 1)
    rows, cols = 3, 512
    w = synth.random_q6k(g, rows, cols)
    x = g.standard_normal((2, cols)).astype(np.float32)
    raw = bytes(w)
    nb = cols // 256
    ref = np.zeros((2, rows))
    for t in range(2):
        for r in range(rows):
            s = 0.0
            for c in range(cols):
                b = r * nb + c // 256
                s += bitwalk_weight(raw[210 * b: 210 * b + 210], c % 256) * float(x[t, c])
            ref[t, r] = s
    assert np.allclose(q6.gemv(w, rows, cols, x), ref, rtol=1e-12, atol=1e-9)


def test_sizes_and_rejects():
    assert q6.q6k_weight_bytes(32000, 4096) == 32000 * 16 * 210
    for bad in ((1, 300), (-1, 256)):
        try:
            q6.q6k_weight_bytes(*bad)
        except ValueError:
            pass
        else:
            raise AssertionError(bad)


def _decode_with(unpack, block):
    """The oracle's dequantisation with another 6-bit unpacker (mutation check)."""
    u = unpack(block[0:128][None], block[128:192][None])[0].astype(np.float64) - 32.0
    sc = block[192:208].view(np.int8).astype(np.float64)
    d = float(np.array([int(block[208]) | (int(block[209]) << 8)], dtype=np.uint16).view(np.float16)[0])
    return d * np.repeat(sc, 16) * u


def test_hand_block_catches_planted_layout_mistakes():
    # each plausible misreading of the layout, planted in a copy of the
    # unpacker, changes at least one hand-derived weight
    h, block = hand_block()
    want = {int(k): v for k, v in h["weights"].items()}

    def swapped_nibbles(ql, qh):      # high nibble for quarters 0-1
        out = q6.unpack_q6(ql, qh).copy()
        for hh in range(2):
            for r in range(4):
                src = ql[..., 64 * hh + 32 * (r % 2): 64 * hh + 32 * (r % 2) + 32]
                low = (src & 0x0F) if r >= 2 else (src >> 4)
                out[..., 128 * hh + 32 * r: 128 * hh + 32 * r + 32] = (out[..., 128 * hh + 32 * r: 128 * hh + 32 * r + 32] & 0x30) | low
        return out

    def reversed_high_bits(ql, qh):   # quarter r takes bits 6-2r, 7-2r
        out = q6.unpack_q6(ql, qh).copy()
        for hh in range(2):
            for r in range(4):
                hi = (qh[..., 32 * hh: 32 * hh + 32] >> (6 - 2 * r)) & 3
                sl = slice(128 * hh + 32 * r, 128 * hh + 32 * r + 32)
                out[..., sl] = (out[..., sl] & 0x0F) | (hi << 4)
        return out

    def ql_quarters_swapped(ql, qh):  # quarter r reads ql[64h + 32(r // 2) + l]
        out = q6.unpack_q6(ql, qh).copy()
        for hh in range(2):
            for r in range(4):
                src = ql[..., 64 * hh + 32 * (r // 2): 64 * hh + 32 * (r // 2) + 32]
                low = (src >> 4) if r >= 2 else (src & 0x0F)
                sl = slice(128 * hh + 32 * r, 128 * hh + 32 * r + 32)
                out[..., sl] = (out[..., sl] & 0x30) | low
        return out

    assert all(_decode_with(q6.unpack_q6, block)[i] == v for i, v in want.items())
    for mutant in (swapped_nibbles, reversed_high_bits, ql_quarters_swapped):
        w = _decode_with(mutant, block)
        assert any(w[i] != v for i, v in want.items()), mutant.__name__
    # a scale per 32 weights instead of 16, and no -32 offset
    w = q6.dequantize(block, 1, 256)[0]
    u = q6.unpack_q6(block[0:128][None], block[128:192][None])[0].astype(np.float64)
    per32 = 0.5 * np.repeat(block[192:208].view(np.int8)[:8].astype(np.float64), 32) * (u - 32)
    no_offset = 0.5 * np.repeat(block[192:208].view(np.int8).astype(np.float64), 16) * u
    assert any(per32[i] != v for i, v in want.items())
    assert any(no_offset[i] != v for i, v in want.items())
    assert all(w[i] == v for i, v in want.items())
