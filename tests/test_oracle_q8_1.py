"""Pins of the oracle's Q8_1 encoding: hand cases, invariants, independent rounding."""
import json
import os

import numpy as np

import bruteforce as bf
from oracle import q4k_oracle as orc
from gemm_block_q4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_blocks():
    with open(os.path.join(GOLDEN, "q8_1_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array([c["x"]], dtype=np.float32)
        q, d16, s = orc.q8_1_quantize(x)
        assert list(q[0]) == c["q"], c["note"]
        assert int(d16.view(np.uint16)[0, 0]) == c["d16_bits"], c["note"]
        assert int(s[0, 0]) == c["sum"], c["note"]


def _mixed_inputs():
    x = synth.activations(21, 16, 1024, outliers=True)
    x[3, 64:96] = 0.0                                   # all-zero block
    x[4, 96:128] = np.float32(1e-30)                    # tiny values
    x[5, 128:160] = np.linspace(-3e4, 3e4, 32, dtype=np.float32)
    x[6, :32] = np.float32(2.0 ** -140)                 # subnormal binary32 inputs
    x[7, 160:192] = np.linspace(-2e7, 9e6, 32, dtype=np.float32)   # saturated scale
    return x


def test_against_independent_scalar_reference():
    x = _mixed_inputs()
    q, d16, s = orc.q8_1_quantize(x)
    for t in range(x.shape[0]):
        for b in range(0, x.shape[1] // 32, 3):
            xs = [float(v) for v in x[t, 32 * b: 32 * b + 32]]
            rq, rd, rs = bf.q8_1_block(xs)
            assert list(q[t, 32 * b: 32 * b + 32]) == rq
            assert float(d16[t, b]) == rd
            assert int(s[t, b]) == rs


def test_invariants():
    x = _mixed_inputs()
    q, d16, s = orc.q8_1_quantize(x)
    m, k = x.shape
    xb = x.reshape(m, k // 32, 32).astype(np.float64)
    qb = q.reshape(m, k // 32, 32).astype(np.int64)
    amax = np.abs(xb).max(-1)
    nz = amax > 0
    assert np.abs(qb).max() <= 127
    # the largest magnitude lands on +-127 in every non-zero block
    assert np.all(np.abs(qb).max(-1)[nz] == 127)
    assert not qb[~nz].any() and not d16[~nz].astype(np.float64).any()
    # odd symmetry
    qn, dn, sn = orc.q8_1_quantize(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d16) and np.array_equal(sn, -s)
    # rounding error at most half a step of the binary32 scale (blocks whose
    # scale is a normal binary32 number; a subnormal scale loses precision and
    # the clamp to 127 can then fire)
    d32 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64)
    normal = (d32 >= 2.0 ** -126) & (d32 < 65520.0)
    err = np.abs(xb - d32[..., None] * qb)
    assert np.all((err <= 0.5 * d32[..., None] * (1 + 2.0 ** -20))[normal])
    # stored sum is the exact integer sum
    assert np.array_equal(s.astype(np.int64), qb.sum(-1))
    # saturated blocks store the largest finite binary16 scale
    sat = d32 >= 65520.0
    assert sat.any() and np.all(d16[sat] == np.float16(65504.0))
    assert np.all(np.isfinite(d16.astype(np.float64)))


def test_exact_ties_round_to_even():
    # d = 2^-3 exactly (amax = 127/8); x = (j + 1/2) * d gives an exact quotient j + 1/2
    d = 2.0 ** -3
    js = np.arange(-40, 40)
    for start in range(0, js.size, 31):
        chunk = js[start:start + 31]
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, 0] = 127 * d
        x[0, 1:1 + chunk.size] = (chunk + 0.5) * d
        q, _, _ = orc.q8_1_quantize(x)
        for i, j in enumerate(chunk):
            want = j if j % 2 == 0 else j + 1
            assert q[0, 1 + i] == want


def test_ds_word_roundtrip():
    x = synth.activations(22, 4, 256, outliers=True)
    _, d16, s = orc.q8_1_quantize(x)
    ds = orc.pack_ds(d16, s)
    d2, s2 = orc.unpack_ds(ds)
    assert np.array_equal(d2.view(np.uint16), d16.view(np.uint16)) and np.array_equal(s2, s)
    assert np.array_equal(ds & 0xFFFF, d16.view(np.uint16))


def test_bf16_input_widening():
    x = synth.activations(23, 2, 128, outliers=True)
    bits = synth.to_bf16_bits(x)
    xf = synth.bf16_bits_to_f32(bits)
    # bf16 values widen exactly and sit within half a bf16 ulp of the f32 draw
    assert np.all(np.abs(xf - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(synth.to_bf16_bits(xf), bits)
