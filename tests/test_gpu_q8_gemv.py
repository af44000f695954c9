"""Q8_1-activation decode GEMV on the GPU against the oracle's reference dot
(normwise bound 1e-5 on identical quantised operands), and against q4k_mmq."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def quantised(m, k, seed):
    return orc.q8_1_quantize(synth.activations(90 + seed, m, k, outliers=True))


def q8_gemv_gpu(q4k, w, qs, d16, s, n, k):
    m = qs.shape[0]
    y = empty((m, n), torch.float32)
    ds = orc.pack_ds(d16, s).view(np.int32)
    q4k.q4k_q8_gemv(dev(w), dev(qs), dev(ds), y, m, n, k)
    return host(y)


def check(q4k, w, qs, d16, s, n, k):
    y = q8_gemv_gpu(q4k, w, qs, d16, s, n, k)
    ref = orc.mmq(w, n, k, qs, d16, s, tokens=list(range(qs.shape[0])))
    xn = np.linalg.norm(orc.q8_1_dequantize(qs, d16), axis=1)
    err = orc.normalized_max_error(y, ref, orc.row_norms(w, n, k), xn)
    assert err <= TOL, err
    return y


# rows narrower than a wavefront (k < 4096), exactly one (4096), spanning
# two, three and eight wavefronts; ragged n; every token-count rounding
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 768), (70, 4096), (33, 8192), (65, 11008), (5, 32768)])
def test_q8_gemv_small(lib, m, n, k):
    say(f"q8 gemv m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(91, 1, n * 7 + k), n, k)
    qs, d16, s = quantised(m, k, n + m)
    check(lib, w, qs, d16, s, n, k)


def test_q8_gemv_integer_special_case_bit_exact(lib):
    # d = 1, sc = 1, dmin = 0 weights and d16 = 1 activations: y is the
    # integer product of the quants, exact in f32 (|y| < 2^24)
    say("q8 gemv integer special case")
    n, k, m = 70, 4608, 8
    rng = np.random.default_rng(92)
    blocks = np.zeros((n * k // 256, 144), dtype=np.uint8)
    blocks[:, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    blocks[:, 4:16] = orc.pack_scale_min(np.ones((1, 8), int), rng.integers(0, 64, (1, 8)))
    blocks[:, 16:] = rng.integers(0, 256, (n * k // 256, 128), dtype=np.uint8)
    qa = rng.integers(-127, 128, (m, k)).astype(np.int8)
    d16 = np.ones((m, k // 32), dtype=np.float16)
    ssum = qa.reshape(m, k // 32, 32).astype(np.int64).sum(-1).astype(np.int16)
    y = q8_gemv_gpu(lib, blocks.reshape(-1), qa, d16, ssum, n, k)
    qw = orc.unpack_quants(blocks[:, 16:]).reshape(n, k).astype(np.int64)
    assert np.array_equal(y.astype(np.float64), (qa.astype(np.int64) @ qw.T).astype(np.float64))


@pytest.mark.parametrize("m,n,k", [(3, 13000, 256), (7, 20000, 512), (2, 300, 16384)])
def test_q8_gemv_many_workgroups(lib, m, n, k):
    # rows per workgroup at their cap of 64 (many workgroups, a ragged last
    # one), and rows spanning four wavefronts
    say(f"q8 gemv m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(94, 1, n + k), n, k)
    qs, d16, s = quantised(m, k, 5)
    check(lib, w, qs, d16, s, n, k)


@pytest.mark.parametrize("m", [1, 4, 8])
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_q8_gemv_sweep_full_size(lib, m, n, k):
    # the three sweep matrices at the token counts bench.py times
    say(f"q8 gemv sweep shape m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(95, 1, n + 7 * k), n, k)
    qs, d16, s = quantised(m, k, 7 + m)
    check(lib, w, qs, d16, s, n, k)


@pytest.mark.parametrize("m,n,k", [(8, 11008, 4096), (4, 4096, 11008)])
def test_q8_gemv_decode_shapes(lib, m, n, k):
    # the 7B-style decode projections, checked against the oracle and against
    # q4k_mmq on the same operands (same product, independent device code)
    say(f"q8 gemv decode shape m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(93, 1, n), n, k)
    qs, d16, s = quantised(m, k, 3)
    y = check(lib, w, qs, d16, s, n, k)
    ym = empty((m, n), torch.float32)
    lib.q4k_mmq(dev(w), dev(qs), dev(orc.pack_ds(d16, s).view(np.int32)), ym, m, n, k)
    ym = host(ym)
    scale = orc.row_norms(w, n, k)[None, :] * np.linalg.norm(orc.q8_1_dequantize(qs, d16), axis=1)[:, None]
    assert np.max(np.abs(y.astype(np.float64) - ym) / scale) <= 2 * TOL
    y2 = q8_gemv_gpu(lib, w, qs, d16, s, n, k)
    assert np.array_equal(y, y2)  # deterministic
