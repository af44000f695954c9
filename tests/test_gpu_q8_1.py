"""Q8_1 quantisation on the GPU is bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu


def mixed(m, k, seed):
    x = synth.activations(60 + seed, m, k, outliers=True)
    if m > 3 and k >= 256:
        x[1, 0:32] = 0.0
        x[2, 32:64] = np.float32(1e-30)
        x[3, 64:96] = np.linspace(-3e4, 3e4, 32, dtype=np.float32)
        x[0, 96:128] = np.float32(-2.0 ** -100)
        x[2, 128:160] = np.linspace(-2e7, 9e6, 32, dtype=np.float32)   # saturated scale
    return x


def run(q4k, x_np, bf16):
    m, k = x_np.shape
    if bf16:
        bits = synth.to_bf16_bits(x_np)
        x = dev(bits.view(np.int16))
        xin = synth.bf16_bits_to_f32(bits)
    else:
        x = dev(x_np)
        xin = x_np
    qs = empty((m, k), torch.int8)
    ds = empty((m, k // 32), torch.int32)
    q4k.q8_1_quantize(x, q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32, m, k, qs, ds)
    return host(qs), host(ds).view(np.uint32), xin


def check(q4k, x_np, bf16):
    qs, ds, xin = run(q4k, x_np, bf16)
    rq, rd, rs = orc.q8_1_quantize(xin)
    assert np.array_equal(qs, rq)
    assert np.array_equal(ds, orc.pack_ds(rd, rs))


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (7, 4096), (33, 768)])
@pytest.mark.parametrize("bf16", [False, True])
def test_q8_1_small(lib, m, k, bf16):
    say(f"q8_1 m={m} k={k} bf16={bf16}")
    check(lib, mixed(m, k, m), bf16)


def test_q8_1_subnormal_binary32_inputs(lib):
    say("q8_1 subnormal inputs")
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :32] = np.float32(2.0 ** -140)
    x[0, 5] = np.float32(3 * 2.0 ** -141)
    x[1, 32:] = np.linspace(-1e-39, 1e-39, 32, dtype=np.float32)
    check(lib, x, False)


def test_q8_1_prefill_activation_bf16(lib):
    say("q8_1 prefill x [512, 5120] bf16")
    x = synth.activations(synth.PREFILL_FFN, 512, 5120, outliers=True, sub=512)
    check(lib, x, True)


def test_q8_1_large_intermediate(lib):
    say("q8_1 intermediate-like values [64, 17408]")
    g = np.random.default_rng(5)
    x = (g.standard_normal((64, 17408)) * g.choice([1.0, 1e3, 1e5], (64, 17408))).astype(np.float32)
    check(lib, x, False)


@pytest.mark.parametrize("bf16", [False, True])
def test_q8_1_exact_ties(lib, bf16):
    # amax = 127 * 2^e, so d = 2^e exactly, and the other values (j + 1/2) 2^e:
    # every quotient is exactly a half-integer and rounds to even (all values
    # have at most 8 significant bits, so bf16 holds them too)
    say(f"q8_1 exact ties bf16={bf16}")
    rng = np.random.default_rng(7)
    m, k = 64, 1024
    e = rng.integers(-10, 10, (m, k // 32, 1)).astype(np.float64)
    j = rng.integers(-126, 126, (m, k // 32, 32)).astype(np.float64)
    x = (j + 0.5) * 2.0 ** e
    x[..., 0] = 127.0 * 2.0 ** e[..., 0]
    check(lib, x.reshape(m, k).astype(np.float32), bf16)
