"""Pins of the oracle's SwiGLU, FFN and MoE compositions."""
import math

import numpy as np
import pytest

import bruteforce as bf
from oracle import q4k_oracle as orc
from gemm_block_q4_amd import synth


def test_silu_closed_forms():
    assert orc.silu(0.0) == 0.0
    assert orc.silu(1.0) == 1.0 / (1.0 + math.exp(-1.0))
    assert abs(orc.silu(1.0) - 0.7310585786300049) < 1e-16      # textbook value
    assert orc.silu(50.0) == 50.0 / (1.0 + math.exp(-50.0))
    assert abs(orc.silu(40.0) - 40.0) < 1e-15
    big_neg = orc.silu(-1000.0)
    assert big_neg == 0.0 and math.copysign(1.0, big_neg) < 0     # -> -0
    g = np.linspace(-20, 20, 101)
    u = np.linspace(3, -3, 101)
    want = [a / (1 + math.exp(-a)) * b for a, b in zip(g, u)]
    assert np.abs(orc.swiglu(g, u) - np.array(want)).max() < 1e-13


def _dense(w, rows, cols):
    return np.array(bf.decode_matrix(bytes(w), rows, cols))


def test_ffn_decode_against_textbook_composition():
    hidden, inter, m = 256, 512, 2
    wg, wu, wd = synth.dense_ffn_weights(41, hidden, inter)
    x = synth.activations(41, m, hidden, outliers=True)
    G, U, D = _dense(wg, inter, hidden), _dense(wu, inter, hidden), _dense(wd, hidden, inter)
    ref = []
    for t in range(m):
        xt = [float(v) for v in x[t]]
        g = [sum(G[i][c] * xt[c] for c in range(hidden)) for i in range(inter)]
        u = [sum(U[i][c] * xt[c] for c in range(hidden)) for i in range(inter)]
        h = [gi / (1 + math.exp(-gi)) * ui if gi > -700 else -0.0 for gi, ui in zip(g, u)]
        ref.append([sum(D[o][i] * h[i] for i in range(inter)) for o in range(hidden)])
    ref = np.array(ref)
    got = orc.ffn_decode(wg, wu, wd, hidden, inter, x)
    assert np.abs(got - ref).max() <= 1e-11 * np.abs(ref).max()


def test_ffn_prefill_is_the_same_ffn_within_quantisation_error():
    hidden, inter, m = 512, 768, 3
    wg, wu, wd = synth.dense_ffn_weights(42, hidden, inter)
    x = synth.activations(42, m, hidden, outliers=False)
    exact = orc.ffn_decode(wg, wu, wd, hidden, inter, x)
    quant = orc.ffn_prefill(wg, wu, wd, hidden, inter, x)
    err = orc.relative_l2(quant, exact)
    assert 1e-5 < err < 3e-2
    # token subsets are exact restrictions (every step is per token)
    sub = orc.ffn_prefill(wg, wu, wd, hidden, inter, x, tokens=[2, 0])
    assert np.array_equal(sub, quant[[2, 0]])


def test_ffn_prefill_steps_by_hand():
    # the prefill composition written out step by step with the scalar Q8_1
    # reference and brute-force dense weights
    hidden, inter, m = 256, 256, 1
    wg, wu, wd = synth.dense_ffn_weights(43, hidden, inter)
    x = synth.activations(43, m, hidden, outliers=True)
    G, U, D = _dense(wg, inter, hidden), _dense(wu, inter, hidden), _dense(wd, hidden, inter)

    def qdq(vec):
        out = []
        for b in range(len(vec) // 32):
            q, d, _ = bf.q8_1_block(vec[32 * b: 32 * b + 32])
            out += [d * v for v in q]
        return out

    xh = qdq([float(v) for v in x[0]])
    g = [sum(G[i][c] * xh[c] for c in range(hidden)) for i in range(inter)]
    u = [sum(U[i][c] * xh[c] for c in range(hidden)) for i in range(inter)]
    h = [bf.f32(gi / (1 + math.exp(-gi)) * ui) if gi > -700 else -0.0 for gi, ui in zip(g, u)]
    hh = qdq(h)
    ref = np.array([sum(D[o][i] * hh[i] for i in range(inter)) for o in range(hidden)])
    got = orc.ffn_prefill(wg, wu, wd, hidden, inter, x)[0]
    assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()


def test_moe_top1_unit_weight_is_the_dense_expert():
    n_exp, hidden, inter, m = 4, 256, 256, 3
    bg, bu, bd = synth.moe_banks(44, n_exp, hidden, inter)
    x = synth.activations(44, m, hidden, outliers=False)
    ids = np.array([[2], [0], [3]], dtype=np.int32)
    wts = np.ones((m, 1), dtype=np.float32)
    y = orc.moe_decode(bg, bu, bd, n_exp, hidden, inter, x, ids, wts)
    gb = orc.q4k_weight_bytes(inter, hidden)
    db = orc.q4k_weight_bytes(hidden, inter)
    for t in range(m):
        e = ids[t, 0]
        ref = orc.ffn_decode(bg[e * gb:(e + 1) * gb], bu[e * gb:(e + 1) * gb],
                             bd[e * db:(e + 1) * db], hidden, inter, x[t:t + 1])
        assert np.array_equal(y[t], ref[0])


def test_moe_is_linear_in_routing_weights():
    n_exp, hidden, inter, m, k = 6, 256, 256, 2, 3
    bg, bu, bd = synth.moe_banks(45, n_exp, hidden, inter)
    x = synth.activations(45, m, hidden, outliers=True)
    ids, wts = synth.router(45, m, n_exp, k)
    y = orc.moe_decode(bg, bu, bd, n_exp, hidden, inter, x, ids, wts)
    parts = 0
    for s in range(k):
        w1 = np.zeros_like(wts)
        w1[:, s] = wts[:, s]
        parts = parts + orc.moe_decode(bg, bu, bd, n_exp, hidden, inter, x, ids, w1)
    assert np.abs(y - parts).max() <= 1e-12 * np.abs(y).max()
    assert np.allclose(wts.sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == k for r in ids.tolist())


def _dequant_pair_ffn(wg, wu, wd, hidden, inter, xt):
    """One pair's prefill FFN from the dequantised matrices and the dequantised
    Q8_1 vectors (plain f64 products, no integer MMQ path)."""
    qx, dx, _ = orc.q8_1_quantize(xt)
    xh = orc.q8_1_dequantize(qx, dx)
    g = xh @ orc.dequantize(wg, inter, hidden).T
    u = xh @ orc.dequantize(wu, inter, hidden).T
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    qh, dh, _ = orc.q8_1_quantize(h)
    return orc.q8_1_dequantize(qh, dh) @ orc.dequantize(wd, hidden, inter).T


def test_moe_prefill_against_dequantised_loops():
    # "micro_moe.rs": one group per (token, selected expert); duplicate experts
    # across tokens, and slots whose expert differs from the slot index
    n_exp, hidden, inter, m, k = 5, 256, 512, 4, 3
    bg, bu, bd = synth.moe_banks(46, n_exp, hidden, inter)
    x = synth.activations(46, m, hidden, outliers=True)
    ids = np.array([[4, 1, 2], [1, 3, 0], [2, 4, 1], [0, 1, 4]], dtype=np.int32)
    wts = np.array([[0.5, 0.25, 0.25], [0.7, 0.2, 0.1], [0.1, 0.1, 0.8], [0.3, 0.3, 0.4]], np.float32)
    y = orc.moe_prefill(bg, bu, bd, n_exp, hidden, inter, x, ids, wts)
    gb = orc.q4k_weight_bytes(inter, hidden)
    db = orc.q4k_weight_bytes(hidden, inter)
    for t in range(m):
        ref = np.zeros(hidden)
        for s in range(k):
            e = ids[t, s]
            ref += float(wts[t, s]) * _dequant_pair_ffn(bg[e * gb:(e + 1) * gb], bu[e * gb:(e + 1) * gb],
                                                         bd[e * db:(e + 1) * db], hidden, inter,
                                                         x[t:t + 1])[0]
        assert np.abs(y[t] - ref).max() <= 1e-9 * np.abs(ref).max()
    # a token subset returns the same rows
    sub = orc.moe_prefill(bg, bu, bd, n_exp, hidden, inter, x, ids, wts, tokens=[3, 1])
    assert np.array_equal(sub, y[[3, 1]])


def test_moe_prefill_top1_is_the_dense_prefill_expert():
    n_exp, hidden, inter, m = 3, 256, 256, 3
    bg, bu, bd = synth.moe_banks(47, n_exp, hidden, inter)
    x = synth.activations(47, m, hidden, outliers=False)
    ids = np.array([[2], [2], [0]], dtype=np.int32)
    wts = np.ones((m, 1), dtype=np.float32)
    y = orc.moe_prefill(bg, bu, bd, n_exp, hidden, inter, x, ids, wts)
    gb = orc.q4k_weight_bytes(inter, hidden)
    db = orc.q4k_weight_bytes(hidden, inter)
    for t in range(m):
        e = ids[t, 0]
        ref = orc.ffn_prefill(bg[e * gb:(e + 1) * gb], bu[e * gb:(e + 1) * gb], bd[e * db:(e + 1) * db],
                              hidden, inter, x[t:t + 1])
        assert np.array_equal(y[t], ref[0])
    with pytest.raises(ValueError):
        orc.moe_prefill(bg, bu, bd, n_exp, hidden, inter, x, np.array([[3], [0], [1]], np.int32), wts)
