"""Decode GEMV on the GPU against the f64 oracle (normwise bound 1e-5)."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def gemv_gpu(q4k, w, x, n, k):
    m = x.shape[0]
    y = empty((m, n), torch.float32)
    q4k.q4k_gemv(dev(w), dev(x), y, m, n, k)
    return host(y)


def check(q4k, w, x, n, k):
    y = gemv_gpu(q4k, w, x, n, k)
    ref = orc.gemv(w, n, k, x)
    err = orc.normalized_max_error(y, ref, orc.row_norms(w, n, k),
                                   np.linalg.norm(x.astype(np.float64), axis=1))
    assert err <= TOL, err
    return y


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(1, 256), (17, 768), (100, 4096), (33, 11008)])
def test_gemv_small(lib, m, n, k):
    say(f"gemv m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(70, 1, n * 7 + k), n, k)
    x = synth.activations(70, m, k, outliers=True, sub=n + m)
    check(lib, w, x, n, k)


@pytest.mark.parametrize("m,n,k", [(3, 5000, 512), (8, 4200, 768), (5, 13000, 256), (2, 16, 32768)])
def test_gemv_multi_token_tiles(lib, m, n, k):
    # 2..8 tokens: two and three 16-row tiles per workgroup, four-wavefront
    # workgroups once the grid exceeds the CUs (13000 rows), and the largest k
    say(f"gemv tiles m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(72, 1, n + k), n, k)
    x = synth.activations(72, m, k, outliers=True, sub=n)
    check(lib, w, x, n, k)


@pytest.mark.parametrize("n,k", [(301, 16384), (77, 20480), (45, 32768)])
def test_gemv_one_token_wide_k(lib, n, k):
    # one token, rows of 64..128 slices: two or four activation units per
    # thread, and the digits of x take more than 64 KiB of LDS from k = 20480
    say(f"gemv one token wide k n={n} k={k}")
    w = synth.random_q4k(synth.rng(73, 1, n + k), n, k)
    x = synth.activations(73, 1, k, outliers=True, sub=n)
    check(lib, w, x, n, k)


@pytest.mark.parametrize("shape", [0, 1, 2])
def test_gemv_sweep_full_size(lib, shape):
    n, k, w, x = synth.gemv_sweep_case(shape)
    say(f"gemv sweep n={n} k={k}")
    y1 = check(lib, w, x, n, k)
    y2 = gemv_gpu(lib, w, x, n, k)
    assert np.array_equal(y1, y2)     # deterministic


def test_gemv_zero_inputs(lib):
    say("gemv zero activation / zero weights")
    n, k = 40, 512
    w = synth.random_q4k(synth.rng(71, 1), n, k)
    y = gemv_gpu(lib, w, np.zeros((2, k), np.float32), n, k)
    assert not y.any()
    w0 = w.copy().reshape(-1, 144)
    w0[:, 0:4] = 0
    y = gemv_gpu(lib, w0.reshape(-1), synth.activations(71, 3, k, False), n, k)
    assert not y.any()
