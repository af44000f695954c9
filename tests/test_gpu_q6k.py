"""Q6_K GEMV (LM head) on the GPU against the Q6_K oracle: normwise error
|y - ref| / (||w_row|| ||x||) <= 1e-5, exact on integer cases."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q6k_oracle as q6
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def gemv_gpu(q4k, w, x, n, k):
    y = empty((n,), torch.float32)
    q4k.q6k_gemv(dev(w), dev(x.reshape(-1)), y, n, k)
    return host(y)


def normwise(y, ref, w, n, k, x):
    scale = q6.row_norms(w, n, k) * np.linalg.norm(x.astype(np.float64))
    return float(np.max(np.abs(y - ref) / np.maximum(scale, 1e-300)))


@pytest.mark.parametrize("n,k", [(1, 256), (3, 768), (37, 4096), (100, 5120), (13, 11008),
                                 (5, 32768), (2047, 1280), (511, 256), (4097, 512)])
def test_q6k_gemv_shapes(lib, n, k):
    say(f"q6k gemv n={n} k={k}")
    w = synth.random_q6k(synth.rng(synth.LM_HEAD, 1, n + k), n, k)
    x = synth.activations(synth.LM_HEAD, 1, k, outliers=True, sub=n + k)
    y = gemv_gpu(lib, w, x, n, k)
    ref = q6.gemv(w, n, k, x)[0]
    assert normwise(y, ref, w, n, k, x) <= TOL


def test_q6k_gemv_integer_case_exact(lib):
    # d = 1, scales = +-1, integer x: every sum is an integer below 2^24, so
    # the f32 result equals the integer product exactly
    say("q6k gemv integer case")
    n, k = 300, 2048
    g = synth.rng(synth.LM_HEAD, 2, 0)
    blocks = synth.random_q6k(g, n, k).reshape(-1, 210)
    blocks[:, 192:208] = g.choice(np.array([1, 255], dtype=np.uint8), (blocks.shape[0], 16))
    blocks[:, 208:210] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    w = blocks.reshape(-1)
    x = g.integers(-3, 4, (1, k)).astype(np.float32)
    y = gemv_gpu(lib, w, x, n, k)
    ref = q6.gemv(w, n, k, x)[0]
    assert np.array_equal(y, ref.astype(np.float32))


def test_q6k_gemv_zero_blocks(lib):
    # d = 0 in every other block and u = 32 in the rest: exact zeros
    say("q6k gemv zero blocks")
    n, k = 64, 1024
    g = synth.rng(synth.LM_HEAD, 3, 0)
    blocks = synth.random_q6k(g, n, k).reshape(-1, 210)
    blocks[::2, 208:210] = 0
    ql, qh = q6.pack_q6(np.full(256, 32, dtype=np.uint8))
    blocks[1::2, :128] = ql
    blocks[1::2, 128:192] = qh
    x = synth.activations(synth.LM_HEAD, 1, k, outliers=True, sub=3)
    assert np.all(gemv_gpu(lib, blocks.reshape(-1), x, n, k) == 0)


def test_q6k_gemv_lm_head_full_size(lib):
    # vocab 32000 x hidden 4096, the launch bench.py times; sampled rows
    # against the oracle, plus determinism
    n, k = 32000, 4096
    say(f"q6k gemv LM head {n}x{k}")
    w, x = synth.lm_head_case(n, k)
    wd, xd = dev(w), dev(x.reshape(-1))
    y1 = empty((n,), torch.float32)
    y2 = empty((n,), torch.float32)
    lib.q6k_gemv(wd, xd, y1, n, k)
    lib.q6k_gemv(wd, xd, y2, n, k)
    y1, y2 = host(y1), host(y2)
    assert np.array_equal(y1, y2)
    rows = np.array([0, 1, 63, 64, 4095, 12345, 31998, 31999])
    rb = q6.q6k_weight_bytes(1, k)
    sub = np.concatenate([w[r * rb:(r + 1) * rb] for r in rows])
    ref = q6.gemv(sub, len(rows), k, x)[0]
    assert normwise(y1[rows], ref, sub, len(rows), k, x) <= TOL
    assert np.all(np.isfinite(y1))
