"""Degenerate inputs on the GPU: all-zero activations and all-zero block scales
give exactly zero outputs on every entry point (the normwise bound of the
other tests says nothing when ||w|| or ||x|| is 0)."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu


def zero_scale_weights(n, k, seed):
    # random quants and 6-bit fields, d = dmin = +0: every weight is 0
    w = synth.random_q4k(synth.rng(96, 1, seed), n, k).reshape(-1, 144).copy()
    w[:, 0:4] = 0
    return w.reshape(-1)


@pytest.mark.parametrize("m,n,k", [(1, 70, 4096), (4, 33, 11008), (8, 5, 256)])
def test_gemv_zero_inputs(lib, m, n, k):
    say(f"gemv zero inputs m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(96, 2, n), n, k)
    for wt, x in ((w, np.zeros((m, k), np.float32)),
                  (zero_scale_weights(n, k, n), synth.activations(96, m, k, outliers=True))):
        y = empty((m, n), torch.float32)
        lib.q4k_gemv(dev(wt), dev(x), y, m, n, k)
        assert not np.any(host(y)), "expected exact zeros"


@pytest.mark.parametrize("entry", ["mmq", "q8_gemv"])
@pytest.mark.parametrize("m,n,k", [(3, 70, 768), (8, 129, 4096)])
def test_q8_products_zero_inputs(lib, entry, m, n, k):
    say(f"{entry} zero inputs m={m} n={n} k={k}")
    w = synth.random_q4k(synth.rng(96, 3, n), n, k)
    zq, zd, zs = orc.q8_1_quantize(np.zeros((m, k), np.float32))  # all-zero blocks: q = d = S = 0
    qs, d16, s = orc.q8_1_quantize(synth.activations(96, m, k, outliers=True))
    fn = lib.q4k_mmq if entry == "mmq" else lib.q4k_q8_gemv
    for wt, (q, d, ss) in ((w, (zq, zd, zs)), (zero_scale_weights(n, k, n), (qs, d16, s))):
        y = empty((m, n), torch.float32)
        fn(dev(wt), dev(q), dev(orc.pack_ds(d, ss).view(np.int32)), y, m, n, k)
        assert not np.any(host(y)), "expected exact zeros"


def test_gemv_multi_token_integer_case_exact(lib):
    # d = 1, sc = 1, dmin = 0 weights and small integer activations: every
    # product and partial sum is an integer far below 2^24, so each path
    # (one-token integer planes, 2-8 token binary16 halves) is exact
    n, k = 40, 1024
    rng = np.random.default_rng(97)
    blocks = np.zeros((n * k // 256, 144), dtype=np.uint8)
    blocks[:, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    blocks[:, 4:16] = orc.pack_scale_min(np.ones((1, 8), int), np.zeros((1, 8), int))
    blocks[:, 16:] = rng.integers(0, 256, (n * k // 256, 128), dtype=np.uint8)
    qw = orc.unpack_quants(blocks[:, 16:]).reshape(n, k).astype(np.int64)
    for m in (1, 3, 8):
        say(f"gemv integer case m={m}")
        x = rng.integers(-50, 51, (m, k)).astype(np.float32)
        y = empty((m, n), torch.float32)
        lib.q4k_gemv(dev(blocks.reshape(-1)), dev(x), y, m, n, k)
        assert np.array_equal(host(y).astype(np.float64), (x.astype(np.int64) @ qw.T).astype(np.float64))
