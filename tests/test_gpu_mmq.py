"""Prefill MMQ on the GPU: bit-exact integer partials, normwise parity 1e-5."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def quantised(m, k, seed, bf16=False):
    x = synth.activations(80 + seed, m, k, outliers=True)
    if bf16:
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    return orc.q8_1_quantize(x)


@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (3, 5, 512), (65, 70, 256), (129, 64, 768)])
def test_partials_bit_exact(lib, m, n, k):
    say(f"mmq partials m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(81, 1, m + n), n, k)
    qs, _, _ = quantised(m, k, m)
    p = empty((m, n, k // 32), torch.int32)
    lib.q4k_test_mmq_partials(dev(w), dev(qs), m, n, k, p)
    assert np.array_equal(host(p).astype(np.int64), orc.mmq_partials(w, n, k, qs))


def mmq_gpu(q4k, w, qs, d16, s, n, k):
    m = qs.shape[0]
    y = empty((m, n), torch.float32)
    ds = orc.pack_ds(d16, s).view(np.int32)
    q4k.q4k_mmq(dev(w), dev(qs), dev(ds), y, m, n, k)
    return host(y)


def test_integer_special_case_bit_exact(lib):
    # d = 1, sc = 1, dmin = 0 weights and d16 = 1 activations: y is the
    # integer product of the quants, exact in f32 (|y| < 2^24)
    say("mmq integer special case")
    n, k, m = 70, 768, 67
    rng = np.random.default_rng(82)
    blocks = np.zeros((n * k // 256, 144), dtype=np.uint8)
    blocks[:, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    blocks[:, 4:16] = orc.pack_scale_min(np.ones((1, 8), int), rng.integers(0, 64, (1, 8)))
    blocks[:, 16:] = rng.integers(0, 256, (n * k // 256, 128), dtype=np.uint8)
    w = blocks.reshape(-1)
    qa = rng.integers(-127, 128, (m, k)).astype(np.int8)
    d16 = np.ones((m, k // 32), dtype=np.float16)
    ssum = qa.reshape(m, k // 32, 32).astype(np.int64).sum(-1).astype(np.int16)
    y = mmq_gpu(lib, w, qa, d16, ssum, n, k)
    qw = orc.unpack_quants(blocks[:, 16:]).reshape(n, k).astype(np.int64)
    assert np.array_equal(y.astype(np.float64), (qa.astype(np.int64) @ qw.T).astype(np.float64))


def check(q4k, w, qs, d16, s, n, k, tokens=None):
    y = mmq_gpu(q4k, w, qs, d16, s, n, k)
    tokens = list(range(qs.shape[0])) if tokens is None else tokens
    ref = orc.mmq(w, n, k, qs, d16, s, tokens=tokens)
    xn = np.linalg.norm(orc.q8_1_dequantize(qs[tokens], d16[tokens]), axis=1)
    err = orc.normalized_max_error(y[tokens], ref, orc.row_norms(w, n, k), xn)
    assert err <= TOL, err
    return y


@pytest.mark.parametrize("m,n,k", [(1, 3, 256), (64, 64, 512), (130, 200, 1024), (7, 129, 2048)])
def test_mmq_small(lib, m, n, k):
    say(f"mmq m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(83, 1, m * 3 + n), n, k)
    qs, d16, s = quantised(m, k, n)
    check(lib, w, qs, d16, s, n, k)


def test_mmq_prefill_gate_full_size(lib):
    n, k, m = 17408, 5120, 512
    say(f"mmq full size m={m} n={n} k={k} (sampled tokens)")
    w = synth.random_q4k(synth.rng(84, 1), n, k)
    qs, d16, s = quantised(m, k, 7, bf16=True)
    # one token from every 128-token tile (a different position in each) and
    # the last one
    tokens = sorted({128 * i + (37 * i + 5) % 128 for i in range(m // 128)} | {0, 63, 64, m - 1})
    y1 = check(lib, w, qs, d16, s, n, k, tokens=tokens)
    y2 = mmq_gpu(lib, w, qs, d16, s, n, k)
    assert np.array_equal(y1, y2)


def test_mmq_down_shape_2048_tokens(lib):
    # the single-matrix MMQ as measured: [5120, 17408] at 2048 tokens (40 x 16
    # workgroups), one token from every 128-token tile and the last
    n, k, m = 5120, 17408, 2048
    say(f"mmq full size m={m} n={n} k={k} (sampled tokens)")
    w = synth.random_q4k(synth.rng(86, 1), n, k)
    qs, d16, s = quantised(m, k, 11, bf16=True)
    tokens = sorted({128 * i + (53 * i + 11) % 128 for i in range(m // 128)} | {m - 1})
    check(lib, w, qs, d16, s, n, k, tokens=tokens)


def test_mmq_max_k(lib):
    # the largest k the prefill path accepts (2^20): the staging offsets of the
    # last blocks and the past-the-end prefetch stay inside 32 bits
    m, n, k = 2, 3, 1 << 20
    say(f"mmq max k m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(85, 1), n, k)
    qs, d16, s = quantised(m, k, 9)
    check(lib, w, qs, d16, s, n, k)
    p = empty((m, n, k // 32), torch.int32)
    lib.q4k_test_mmq_partials(dev(w), dev(qs), m, n, k, p)
    assert np.array_equal(host(p).astype(np.int64), orc.mmq_partials(w, n, k, qs))


def bf16_rne(y32):
    """bfloat16 bits of finite f32 values, rounded to nearest even (numpy)."""
    b = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (3, 300, 512), (130, 520, 1024), (257, 64, 768),
                                   (512, 5120, 17408)])
def test_mmq_bf16_store(lib, m, n, k):
    # the bf16 store is the nearest-even rounding of the f32 result, bit for
    # bit; against the oracle it is within half a bf16 unit plus the f32 bound
    say(f"mmq bf16 store m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(84, 1, m + n + k), n, k)
    x = synth.activations(84, m, k, outliers=True, sub=m + n)
    qs, d16, s = orc.q8_1_quantize(x)
    ds = orc.pack_ds(d16, s).view(np.int32)
    wd, qd, dd = dev(w), dev(qs), dev(ds)
    y32 = empty((m, n), torch.float32)
    y16 = empty((m, n), torch.int16)
    lib.q4k_mmq(wd, qd, dd, y32, m, n, k)
    lib.q4k_mmq_bf16(wd, qd, dd, y16, m, n, k)
    y32, y16 = host(y32), host(y16).view(np.uint16)
    assert np.array_equal(y16, bf16_rne(y32))
    tokens = [0, m - 1] if m * n * k > 1 << 28 else list(range(m))
    ref = orc.mmq(w, n, k, qs[tokens], d16[tokens], s[tokens])
    got = synth.bf16_bits_to_f32(y16[tokens]).astype(np.float64)
    bound = np.abs(ref) * 2.0 ** -8 + 1e-5 * orc.row_norms(w, n, k)[None, :] * \
        np.linalg.norm(orc.q8_1_dequantize(qs[tokens], d16[tokens]), axis=1)[:, None]
    assert np.all(np.abs(got - ref) <= bound)
