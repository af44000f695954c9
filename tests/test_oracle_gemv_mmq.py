"""Pins of the oracle's GEMV and reference dot (MMQ) against brute force and
closed forms."""
import numpy as np
import pytest

import bruteforce as bf
from oracle import q4k_oracle as orc
from gemm_block_q4_amd import synth


@pytest.mark.parametrize("n,k,m", [(1, 256, 1), (3, 512, 2), (7, 256, 8), (2, 768, 3)])
def test_gemv_against_python_loops(n, k, m):
    w = synth.random_q4k(synth.rng(31, 1, n * 1000 + k), n, k)
    x = synth.activations(31, m, k, outliers=True, sub=n)
    mat = bf.decode_matrix(bytes(w), n, k)
    xs = [[float(v) for v in row] for row in x]
    ref = np.array([[sum(mat[j][i] * xs[t][i] for i in range(k)) for j in range(n)]
                    for t in range(m)])
    got = orc.gemv(w, n, k, x)
    scale = np.abs(ref).max() + 1
    assert np.abs(got - ref).max() <= 1e-13 * scale


def _q8(x):
    q = []
    d = []
    s = []
    for row in x:
        qr, dr, sr = [], [], []
        for b in range(len(row) // 32):
            qb, db, sb = bf.q8_1_block([float(v) for v in row[32 * b: 32 * b + 32]])
            qr += qb
            dr.append(db)
            sr.append(sb)
        q.append(qr)
        d.append(dr)
        s.append(sr)
    return q, d, s


def test_partials_against_python_loops():
    n, k, m = 3, 512, 2
    w = synth.random_q4k(synth.rng(32, 1), n, k)
    x = synth.activations(32, m, k, outliers=True)
    q, _, _ = _q8(x)
    blocks = bytes(w)
    ref = np.zeros((m, n, k // 32), dtype=np.int64)
    for t in range(m):
        for j in range(n):
            for b in range(k // 256):
                blk = blocks[(j * (k // 256) + b) * 144:(j * (k // 256) + b + 1) * 144]
                for i in range(256):
                    ref[t, j, 8 * b + i // 32] += bf.quant_bitwalk(blk[16:], i) * q[t][256 * b + i]
    qs, _, _ = orc.q8_1_quantize(x)
    assert np.array_equal(orc.mmq_partials(w, n, k, qs), ref)


def test_refdot_against_python_loops():
    n, k, m = 2, 512, 2
    w = synth.random_q4k(synth.rng(33, 1), n, k)
    x = synth.activations(33, m, k, outliers=True)
    q, d, s = _q8(x)
    mat = bf.decode_matrix(bytes(w), n, k)
    # dequantise-then-dot: the reference dot equals sum_k w_hat * x_hat with
    # x_hat = d16 * q (the integer block sum makes the min term exact)
    ref = np.array([[sum(mat[j][i] * d[t][i // 32] * q[t][i] for i in range(k))
                     for j in range(n)] for t in range(m)])
    qs, d16, ss = orc.q8_1_quantize(x)
    got = orc.mmq(w, n, k, qs, d16, ss)
    assert np.abs(got - ref).max() <= 1e-12 * (np.abs(ref).max() + 1)


def test_refdot_integer_special_case():
    # d = 1, every sc = 1, dmin = 0 and a Q8_1 operand with d16 = 1 reduce the
    # reference dot to a plain integer matrix product
    n, k, m = 5, 768, 4
    rng = np.random.default_rng(34)
    blocks = np.zeros((n * k // 256, 144), dtype=np.uint8)
    blocks[:, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    blocks[:, 4:16] = orc.pack_scale_min(np.ones((1, 8), int), rng.integers(0, 64, (1, 8)))
    blocks[:, 16:] = rng.integers(0, 256, (n * k // 256, 128), dtype=np.uint8)
    w = blocks.reshape(-1)
    qa = rng.integers(-127, 128, (m, k)).astype(np.int8)
    d16 = np.ones((m, k // 32), dtype=np.float16)
    ssum = qa.reshape(m, k // 32, 32).astype(np.int64).sum(-1).astype(np.int16)
    qw = orc.unpack_quants(blocks[:, 16:]).reshape(n, k).astype(np.int64)
    ref = qa.astype(np.int64) @ qw.T
    got = orc.mmq(w, n, k, qa, d16, ssum)
    assert np.array_equal(got, ref.astype(np.float64))


def test_refdot_matches_gemv_on_dequantised_activations():
    n, k, m = 9, 1024, 3
    w = synth.random_q4k(synth.rng(35, 1), n, k)
    x = synth.activations(35, m, k, outliers=True)
    qs, d16, ss = orc.q8_1_quantize(x)
    xhat = orc.q8_1_dequantize(qs, d16)
    a = orc.mmq(w, n, k, qs, d16, ss)
    b = orc.gemv(w, n, k, xhat.astype(np.float32))   # x_hat is exact in f32
    assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


def test_token_subset_equals_full():
    n, k, m = 4, 512, 6
    w = synth.random_q4k(synth.rng(36, 1), n, k)
    x = synth.activations(36, m, k, outliers=False)
    qs, d16, ss = orc.q8_1_quantize(x)
    full = orc.mmq(w, n, k, qs, d16, ss)
    sub = orc.mmq(w, n, k, qs, d16, ss, tokens=[5, 1])
    assert np.array_equal(sub, full[[5, 1]])


def test_error_metrics():
    y = np.array([[1.0, 2.0]])
    assert orc.normalized_max_error(y, y, np.array([1.0, 1.0]), np.array([1.0])) == 0.0
    assert orc.normalized_max_error(y + 1e-3, y, np.array([2.0, 4.0]), np.array([0.5])) == pytest.approx(1e-3)
    # a zero denominator demands an exact zero
    assert orc.normalized_max_error(np.array([[1e-30]]), np.array([[0.0]]), np.array([0.0]),
                                    np.array([1.0])) == float("inf")
    assert orc.relative_l2(np.array([3.0, 4.0]) * 1.001, np.array([3.0, 4.0])) == pytest.approx(1e-3)
