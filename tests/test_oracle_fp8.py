"""Pins of the FP8 (E4M3) prefill-recipe oracle ("fp8_recipe.rs").

Checked against the format's definition rather than the oracle's own
formulas: a decode table written from the E4M3FN definition, a brute-force
nearest-value search over all finite codes (ties to the even code), codes
derived by hand, the page's saturation and subnormal rules, and the GEMM
against Python loops over the decoded values."""
import itertools
import math

import numpy as np
import pytest

from oracle import fp8_oracle as fp8


def definition_value(code: int) -> float:
    """E4M3FN from the format definition (sign, 4-bit exponent bias 7, 3-bit
    mantissa; exponent 0 subnormal; 0x7F/0xFF NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


def test_decode_matches_definition_and_hand_values():
    codes = np.arange(256, dtype=np.uint8)
    got = fp8.e4m3_decode(codes)
    for c in range(256):
        want = definition_value(c)
        assert (math.isnan(want) and math.isnan(got[c])) or got[c] == want, c
    hand = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x40: 2.0, 0x3F: 1.875,
            0x37: 0.9375, 0x2A: 0.3125, 0x58: 16.0, 0xB8: -1.0}
    for c, v in hand.items():
        assert got[c] == v, hex(c)
    assert got[0x80] == 0.0 and math.copysign(1.0, got[0x80]) == -1.0


def brute_encode(v: float) -> int:
    """Nearest finite E4M3 value by exhaustive search, ties to the even code
    (even mantissa); |v| beyond 448 saturates; zero keeps its sign."""
    a = min(abs(v), 448.0)
    best, best_d = None, None
    for c in range(0x7F):  # positive finite codes 0x00 .. 0x7E
        d = abs(definition_value(c) - a)
        if best is None or d < best_d or (d == best_d and (c & 1) == 0):
            best, best_d = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_encode_matches_brute_force_search():
    rng = np.random.default_rng(5)
    vals = [0.0, -0.0, 448.0, -448.0, 1000.0, 464.0, 463.9, 480.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10,
            3 * 2.0 ** -10, 15.5, 0.3, 1.0625, 1.1875, 2.0 ** -7 + 2.0 ** -11, 1e-30]
    # every midpoint between adjacent codes, and its neighbours in binary32
    pos = [definition_value(c) for c in range(0x7F)]
    for lo, hi in zip(pos, pos[1:]):
        mid = np.float32((lo + hi) / 2)
        vals += [float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9)))]
    vals += list(rng.normal(0, 50, 400).astype(np.float32)) + list(rng.normal(0, 0.01, 200).astype(np.float32))
    v = np.array(vals, dtype=np.float32)
    got = fp8.e4m3_encode(v)
    want = np.array([brute_encode(float(x)) for x in v], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_encode_hand_codes():
    # derived by hand from the definition
    cases = {
        0.3: 0x2A,          # 1.2 * 2^-2: significand 9.6 -> 10 -> mantissa 2, exponent 5
        1000.0: 0x7E,       # saturates at 448
        -0.001: 0x81,       # subnormal: 0.512 -> 1 -> -2^-9
        2.0 ** -10: 0x00,   # subnormal tie 0.5 -> 0 (even)
        3 * 2.0 ** -10: 0x02,  # subnormal tie 1.5 -> 2 (even)
        15.5: 0x58,         # significand tie 15.5 -> 16: carry to 2^4, mantissa 0
        224.0: 0x76,        # 1.75 * 2^7
        -448.0: 0xFE,
        112.0: 0x6E,        # 1.75 * 2^6
    }
    v = np.array(list(cases.keys()), dtype=np.float32)
    got = fp8.e4m3_encode(v)
    for x, c, g in zip(cases.keys(), cases.values(), got):
        assert g == c, (x, hex(g), hex(c))


def test_planted_encoder_mistakes_fail_the_hand_codes():
    v = np.array([-0.001, 2.0 ** -10, 3 * 2.0 ** -10, 15.5, 1000.0], dtype=np.float32)
    want = np.array([0x81, 0x00, 0x02, 0x58, 0x7E], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(v), want)
    flushed = np.where(np.abs(v) < 2.0 ** -6, 0, fp8.e4m3_encode(v)).astype(np.uint8)   # subnormals to zero
    assert not np.array_equal(flushed, want)
    away = np.array([brute_encode(float(np.sign(x) * (abs(x) + 1e-7))) for x in v], dtype=np.uint8)  # ties up
    assert not np.array_equal(away, want)


def test_absmax_and_quantize_rows_hand_row():
    x = np.array([[1.0, -2.0, 0.5, 0.0], [0.0, 0.0, 0.0, 0.0], [3.0, 0.0, -1.5, 0.75]], np.float32)
    q, am = fp8.quantize_rows(x)
    assert list(am) == [2.0, 0.0, 3.0]
    # row 0: scale 448 / 2 = 224: [224, -448, 112, 0]
    assert list(q[0]) == [0x76, 0xFE, 0x6E, 0x00]
    # zero row: absmax 0 taken as 1, every code 0
    assert not np.any(q[1])
    # row 2: scale 448/3 = 149.333.. (binary32); 3 -> 448, -1.5 -> -224, 0.75 -> 112
    assert list(q[2]) == [0x7E, 0x00, 0xF6, 0x6E]


def test_gemm_against_python_loops():
    rng = np.random.default_rng(6)
    m, n, k = 3, 4, 64
    a = rng.normal(0, 1, (m, k)).astype(np.float32)
    a[1, 5] = 80.0
    w = rng.normal(0, 0.1, (n, k)).astype(np.float32)
    w[2] = 0.0
    qa, aa = fp8.quantize_rows(a)
    qw, wa = fp8.quantize_rows(w)
    y = fp8.gemm_rows(qa, aa, qw, wa)
    for t, c in itertools.product(range(m), range(n)):
        d = sum(definition_value(int(qa[t, i])) * definition_value(int(qw[c, i])) for i in range(k))
        d32 = np.float32(d)
        b = int(d32.view(np.uint32))
        b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
        db = np.uint32(b).view(np.float32)
        f1 = np.float32(aa[t] if aa[t] != 0 else 1) / np.float32(448)
        f2 = np.float32(wa[c] if wa[c] != 0 else 1) / np.float32(448)
        want = np.float32(np.float32(db * f1) * f2)
        assert y[t, c] == want, (t, c)
    # the recipe approximates x . w: relative error of a per-row E4M3 product
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    err = np.abs(y - exact)
    assert np.all(err <= 0.1 * np.linalg.norm(a, axis=1)[:, None] * np.linalg.norm(w, axis=1)[None, :] + 1e-12)


def test_dequant_outer_hand_values():
    # "fp8_recipe.rs", fp8_dequant_outer: D rounded to BF16, times a/448, times w/448
    D = np.array([[1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0]])
    y = fp8.dequant_outer(D, np.array([448.0], np.float32), np.array([448.0, 0.0, 896.0, 224.0], np.float32))
    # 1 + 2^-8 is the tie between 1 and 1 + 2^-7: even mantissa (1); 1 + 3 2^-8
    # the tie between 1 + 2^-7 and 1 + 2^-6: even mantissa (1 + 2^-6)
    assert y[0, 0] == np.float32(1.0)
    assert y[0, 1] == np.float32(1.0) / np.float32(448.0)       # zero absmax taken as 1
    assert y[0, 2] == np.float32(1.015625) * np.float32(2.0)
    assert y[0, 3] == np.float32(-1.5)
    # both factors applied: a = 224 halves every output
    y2 = fp8.dequant_outer(D, np.array([224.0], np.float32), np.array([448.0, 448.0, 448.0, 448.0], np.float32))
    assert list(y2[0]) == [0.5, 0.5, np.float32(1.015625) / 2, -1.5]
    # the binary32 product order: (D * f1) * f2 with f1 = 3/448, f2 = 5/448
    d = np.float32(1.5)
    f1 = np.float32(3.0) / np.float32(448.0)
    f2 = np.float32(5.0) / np.float32(448.0)
    y3 = fp8.dequant_outer(np.array([[1.5]]), np.array([3.0], np.float32), np.array([5.0], np.float32))
    assert y3[0, 0] == np.float32(np.float32(d * f1) * f2)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([np.inf], np.float32))
