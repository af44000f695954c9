"""Pins of the oracle's acceptance denominators and of the quantiser's binary16
saturation, on hand-built inputs whose expected values were worked out by hand.

``row_norms`` is the ||w_hat_n|| in every normwise GEMV/MMQ/Q6_K bound
(max |err| / (||w_n|| ||x_t||)), so a mistake in it loosens every parity test
silently.  The hand matrices are non-square and also embedded in a square one,
so that a dropped square root, a reduction over the wrong axis, or an L1 / max
norm in place of the Euclidean one each change a hand-derived value.

The quantiser's scale saturation ("q4k_mmq.rs", quantize_weight_q4k stores
fp16 d and dmin; the pages say nothing of overflow, and the reading taken is
65504 wherever the round-to-nearest-even conversion would give infinity) is
pinned by blocks whose step and offset reach the binary16 overflow point, with
every code derived by hand.
"""
import math

import numpy as np

from oracle import q4k_oracle as orc
from oracle import q6k_oracle as q6


# -- Q4_K row norms ----------------------------------------------------------------

def q4k_hand_matrix():
    """3 rows x 512 columns (two blocks per row) of block_q4_K, built byte by byte.

    Layout (GGML block_q4_K): d bytes 0-1, dmin 2-3, scales 4-15, quants 16-143;
    sub-blocks 0-3 take sc from the low 6 bits of scales[j] and m from the low 6
    bits of scales[j+4]; sub-blocks 4-7 take the low 4 bits from scales[j+4]
    (sc: low nibble, m: high nibble) and the high 2 bits from the top of
    scales[j-4] (sc) and scales[j] (m).  Weight 64g+l is the low nibble of quant
    byte 32g+l, weight 64g+32+l its high nibble.

    Row 0, block 0: d = 1.0 (0x3C00), dmin = 0.5 (0x3800), scales[0] = 2 (sc_0
      = 2), scales[4] = 1 (m_0 = 1); quant byte 0 = 0x01 (weight 0: q = 1).
      Weights 0..31: 1*2*q - 0.5*1, i.e. 1.5 for weight 0 and -0.5 for the
      other 31.  Sub-blocks 1..7 have sc = m = 0.  Block 1 all zero bytes.
      ||w||^2 = 2.25 + 31 * 0.25 = 10.
    Row 1, block 1: d = 1.0, dmin = 0, scales[8] = 0x03 (sc_4 = 3, m_4 = 0);
      quant byte 64 = 0x03 (weight 128: q = 3), byte 65 = 0x04 (weight 129:
      q = 4).  Weights 128, 129 of the block (columns 384, 385) = 9, 12; every
      other weight 0.  ||w|| = 15.
    Row 2, block 0: d = 0, dmin = 0.25 (0x3400), scales[11] = 0xF0 and
      scales[7] = 0xC0 (m_7 = 15 | 3 << 4 = 63; sc_3 = m_3 = 0).  Weights
      224..255 = -0.25 * 63 = -15.75, every other weight 0 (d = 0).
      ||w||^2 = 32 * 15.75^2 = 7938 = 2 * 63^2, ||w|| = 63 * sqrt(2).
    """
    w = np.zeros((3, 2, 144), dtype=np.uint8)
    # row 0, block 0
    w[0, 0, 0:2] = (0x00, 0x3C)
    w[0, 0, 2:4] = (0x00, 0x38)
    w[0, 0, 4 + 0] = 2
    w[0, 0, 4 + 4] = 1
    w[0, 0, 16 + 0] = 0x01
    # row 1, block 1
    w[1, 1, 0:2] = (0x00, 0x3C)
    w[1, 1, 4 + 8] = 0x03
    w[1, 1, 16 + 64] = 0x03
    w[1, 1, 16 + 65] = 0x04
    # row 2, block 0
    w[2, 0, 2:4] = (0x00, 0x34)
    w[2, 0, 4 + 11] = 0xF0
    w[2, 0, 4 + 7] = 0xC0
    want = np.array([math.sqrt(10.0), 15.0, 63.0 * math.sqrt(2.0)])
    return w.reshape(-1), want


def test_q4k_hand_matrix_weights():
    # the dequantised weights the norms are derived from
    w, _ = q4k_hand_matrix()
    dq = orc.dequantize(w, 3, 512)
    assert dq[0, 0] == 1.5 and np.all(dq[0, 1:32] == -0.5) and not np.any(dq[0, 32:])
    assert dq[1, 384] == 9.0 and dq[1, 385] == 12.0
    assert np.count_nonzero(dq[1]) == 2
    assert np.all(dq[2, 224:256] == -15.75) and np.count_nonzero(dq[2]) == 32


def test_q4k_row_norms_hand_values():
    w, want = q4k_hand_matrix()
    got = orc.row_norms(w, 3, 512)
    assert got.shape == (3,)
    assert np.allclose(got, want, rtol=1e-15, atol=0)


def square_embedding(w_rows, rows_used, cols):
    """The hand rows (one block wide each) as the first rows of a square
    256 x 256 matrix, the other rows zero."""
    out = np.zeros((256, 1, 144), dtype=np.uint8)
    out[:rows_used, 0] = np.asarray(w_rows, dtype=np.uint8).reshape(rows_used, cols // 256, 144)[:, 0]
    return out.reshape(-1)


def test_q4k_row_norms_square_matrix():
    # block 0 of each hand row: row 0 keeps its norm sqrt(10), row 1 is zero
    # there (its weights sit in block 1), row 2 keeps 63 sqrt(2)
    w, _ = q4k_hand_matrix()
    sq = square_embedding(w, 3, 512)
    got = orc.row_norms(sq, 256, 256)
    want = np.zeros(256)
    want[0] = math.sqrt(10.0)
    want[2] = 63.0 * math.sqrt(2.0)
    assert np.allclose(got, want, rtol=1e-15, atol=0)


def test_q4k_row_norms_catch_planted_mistakes():
    # each plausible mistake in the norm, planted in a copy, changes at least
    # one hand-derived value (non-square and square matrices)
    w, want = q4k_hand_matrix()
    sq = square_embedding(w, 3, 512)
    want_sq = np.zeros(256)
    want_sq[0] = math.sqrt(10.0)
    want_sq[2] = 63.0 * math.sqrt(2.0)
    mutants = {
        "no sqrt": lambda a, r, c: (orc.dequantize(a, r, c) ** 2).sum(axis=1),
        "wrong axis": lambda a, r, c: np.sqrt((orc.dequantize(a, r, c) ** 2).sum(axis=0)),
        "L1 norm": lambda a, r, c: np.abs(orc.dequantize(a, r, c)).sum(axis=1),
        "max norm": lambda a, r, c: np.abs(orc.dequantize(a, r, c)).max(axis=1),
        "no min term": lambda a, r, c: np.sqrt((_dequant_no_min(a, r, c) ** 2).sum(axis=1)),
    }

    def passes(fn, a, r, c, expect):
        got = np.asarray(fn(a, r, c))
        return got.shape == expect.shape and np.allclose(got, expect, rtol=1e-15, atol=0)

    assert passes(orc.row_norms, w, 3, 512, want) and passes(orc.row_norms, sq, 256, 256, want_sq)
    for name, fn in mutants.items():
        assert not passes(fn, w, 3, 512, want), name
        assert not passes(fn, sq, 256, 256, want_sq), name


def _dequant_no_min(w, rows, cols):
    d, _, sc, _, q = orc.block_fields(w, rows, cols)
    return (d[..., None] * np.repeat(sc, 32, axis=-1) * q).reshape(rows, cols)


# -- Q6_K row norms ----------------------------------------------------------------

def q6k_hand_matrix():
    """2 rows x 512 columns of block_q6_K (210 bytes: ql 0-127, qh 128-191,
    int8 scales 192-207, binary16 d 208-209), built byte by byte.

    Every weight starts at u = 32 (low 4 bits 0, high 2 bits 2: every qh byte
    0xAA holds 2 in each of its four 2-bit fields), so w = d*scale*(u-32) = 0.

    Row 0, block 0: d = 1.0 (0x3C00), scales[0] = 1; ql[0] = 0x03 (weight 0:
      u = 35), ql[1] = 0x04 (weight 1: u = 36).  Weights 0, 1 = 3, 4;
      ||w|| = 5.
    Row 1, block 1: d = 0.5 (0x3800), scales[15] = -2 (0xFE); weight 255 is
      half 1, quarter 3, l = 31: the high nibble of ql[64 + 32 + 31] = ql[127]
      (0) and bits 6-7 of qh[32 + 31] = qh[63], set to 0 (qh[63] = 0x2A), so
      u = 0 and the weight is 0.5 * -2 * -32 = 32; weight 254 likewise with
      ql[126] = 0x10 (high nibble 1) and qh[62] = 0x2A: u = 1, weight
      0.5 * -2 * -31 = 31.  ||w||^2 = 32^2 + 31^2 = 1985.
    """
    w = np.zeros((2, 2, 210), dtype=np.uint8)
    w[..., 128:192] = 0xAA
    w[0, 0, 208:210] = (0x00, 0x3C)
    w[0, 0, 192] = 1
    w[0, 0, 0] = 0x03
    w[0, 0, 1] = 0x04
    w[1, 1, 208:210] = (0x00, 0x38)
    w[1, 1, 192 + 15] = 0xFE
    w[1, 1, 127] = 0x00
    w[1, 1, 128 + 63] = 0x2A
    w[1, 1, 126] = 0x10
    w[1, 1, 128 + 62] = 0x2A
    want = np.array([5.0, math.sqrt(1985.0)])
    return w.reshape(-1), want


def test_q6k_hand_matrix_weights():
    w, _ = q6k_hand_matrix()
    dq = q6.dequantize(w, 2, 512)
    assert dq[0, 0] == 3.0 and dq[0, 1] == 4.0 and np.count_nonzero(dq[0]) == 2
    assert dq[1, 511] == 32.0 and dq[1, 510] == 31.0 and np.count_nonzero(dq[1]) == 2


def test_q6k_row_norms_hand_values_and_planted_mistakes():
    w, want = q6k_hand_matrix()
    got = q6.row_norms(w, 2, 512)
    assert got.shape == (2,) and np.allclose(got, want, rtol=1e-15, atol=0)
    mutants = {
        "no sqrt": lambda a, r, c: (q6.dequantize(a, r, c) ** 2).sum(axis=1),
        "wrong axis": lambda a, r, c: np.linalg.norm(q6.dequantize(a, r, c), axis=0),
        "L1 norm": lambda a, r, c: np.abs(q6.dequantize(a, r, c)).sum(axis=1),
        "max norm": lambda a, r, c: np.abs(q6.dequantize(a, r, c)).max(axis=1),
    }
    for name, fn in mutants.items():
        g = np.asarray(fn(w, 2, 512))
        assert g.shape != want.shape or not np.allclose(g, want, rtol=1e-15, atol=0), name


def test_normalized_max_error_hand_values():
    # |y - y_ref| / (||w_n|| ||x_t||) with hand numbers: errors 0.5 and 3 over
    # denominators 2*5 and 2*15 (and a zero row with y exactly 0)
    y_ref = np.array([[1.0, 2.0, 0.0]])
    y = np.array([[1.5, 5.0, 0.0]])
    got = orc.normalized_max_error(y, y_ref, np.array([5.0, 15.0, 0.0]), np.array([2.0]))
    assert got == max(0.5 / 10.0, 3.0 / 30.0)
    # a non-zero result where the denominator is 0 is an infinite error
    assert orc.normalized_max_error(np.array([[0.0, 0.0, 1e-30]]), y_ref * 0, np.array([5.0, 15.0, 0.0]),
                                    np.array([2.0])) == float("inf")


# -- quantiser: binary16 saturation of d and dmin ----------------------------------

def test_quantizer_saturates_d_and_dmin_hand_codes():
    """One block: sub-block 0 = {0 (31 times), 66150000}, sub-block 1 =
    {0 (31 times), -4410000}, sub-blocks 2..7 all zero.  Every value and step
    below is exact in binary32.

    sub-block 0: lo = 0, hi = 66150000, o = 0, s = 66150000 / 15 = 4410000
    sub-block 1: lo = -4410000, hi = 0, o = 4410000, s = 4410000 / 15 = 294000
    d = f16(4410000 / 63) = f16(70000) -> overflow -> 65504 (0x7BFF)
    dmin = f16(4410000 / 63) = f16(70000) -> 65504 (0x7BFF)
    sc_0 = rint(4410000 / 65504) = rint(67.32..) -> clamped to 63
    sc_1 = rint(294000 / 65504) = rint(4.488..) = 4;  m_0 = 0
    m_1 = rint(4410000 / 65504) -> clamped to 63
    codes: d*sc_0 = 4126752, sub-block 0 adds dmin*m_0 = 0:
      q(66150000) = rint(16.03..) -> 15;  q(0) = 0
    d*sc_1 = 262016, sub-block 1 adds dmin*m_1 = 4126752:
      q(-4410000) = rint(-283248 / 262016) = rint(-1.08..) -> clamped to 0
      q(0) = rint(4126752 / 262016) = rint(15.75) = 16 -> clamped to 15
    """
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, 5] = 66150000.0
    x[0, 32 + 7] = -4410000.0
    b = orc.q4k_quantize(x)
    assert b.size == 144
    assert (int(b[0]) | int(b[1]) << 8) == 0x7BFF      # d = 65504
    assert (int(b[2]) | int(b[3]) << 8) == 0x7BFF      # dmin = 65504
    sc, mn = orc.unpack_scale_min(b[4:16])
    assert list(sc) == [63, 4, 0, 0, 0, 0, 0, 0]
    assert list(mn) == [0, 63, 0, 0, 0, 0, 0, 0]
    q = orc.unpack_quants(b[16:144])
    want = np.zeros(256, dtype=np.uint8)
    want[5] = 15
    want[32:64] = 15
    want[32 + 7] = 0
    assert np.array_equal(q, want)
    # a plain (non-saturating) binary16 conversion would store infinity
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(np.float64(70000.0)))


def test_quantizer_saturation_threshold_is_the_rounding_tie():
    """s / 63 exactly 65520 (the tie between 65504 and 2^16, which rounds to
    even, i.e. to infinity) saturates; s / 63 = 65519 rounds to 65504 without
    saturation; 65472 is the next binary16 below and stays.

    hi - lo = 65520 * 63 * 15 = 61916400 -> s = 4127760 -> s/63 = 65520
    hi - lo = 65519 * 63 * 15 = 61915455 is not exact in binary32 (odd, above
    2^24), so the second case uses hi = 65472 * 945 = 61871040 (exact), whose
    step is 4124736 and s/63 = 65472 exactly.
    """
    x = np.zeros((3, 256), dtype=np.float32)
    x[0, 0] = 61916400.0
    x[1, 0] = 61871040.0
    x[2, 0] = -61916400.0     # the same through the offset: o = 61916400, dmin saturates
    b = orc.q4k_quantize(x).reshape(3, 144)
    d = [int(r[0]) | int(r[1]) << 8 for r in b]
    dmin = [int(r[2]) | int(r[3]) << 8 for r in b]
    assert d[0] == 0x7BFF                              # 65520 -> saturated to 65504
    assert d[1] == int(np.float16(65472.0).view(np.uint16))   # 0x7BFE, exact
    assert dmin[0] == 0 and dmin[1] == 0
    # row 2: lo = -61916400, hi = 0: o / 63 = 982800 -> saturated; s the same
    # span over 15 -> s / 63 = 65520 -> saturated
    assert dmin[2] == 0x7BFF and d[2] == 0x7BFF
    # the planted mistake "convert without saturating" gives infinity there
    with np.errstate(over="ignore"):
        assert int(np.float16(np.float64(65520.0)).view(np.uint16)) == 0x7C00
