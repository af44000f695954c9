"""Load-time Q4_K quantiser on the GPU: bit-exact bytes against the oracle."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu


def quantize_gpu(q4k, x, rows, cols, bf16=False):
    w = empty((q4k.q4k_weight_bytes(rows, cols),), torch.uint8)
    src = dev(synth.to_bf16_bits(x).view(np.int16)) if bf16 else dev(x)
    q4k.q4k_quantize(src, q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32, rows, cols, w)
    return host(w)


@pytest.mark.parametrize("rows,cols,outliers", [(1, 256, False), (3, 768, True), (37, 4096, True),
                                                (130, 11008, False)])
def test_quantize_bit_exact(lib, rows, cols, outliers):
    say(f"q4k quantize rows={rows} cols={cols}")
    x = synth.activations(98, rows, cols, outliers=outliers, sub=rows)
    assert np.array_equal(quantize_gpu(lib, x, rows, cols), orc.q4k_quantize(x))


@pytest.mark.parametrize("rows,cols", [(5, 512), (64, 2048), (3, 768), (1, 256)])
def test_quantize_bf16_bit_exact(lib, rows, cols):
    say(f"q4k quantize bf16 rows={rows} cols={cols}")
    x = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.activations(99, rows, cols, outliers=True)))
    assert np.array_equal(quantize_gpu(lib, x, rows, cols, bf16=True), orc.q4k_quantize(x))


def test_quantize_special_values(lib):
    # zero blocks (of both zero signs), constant and all-negative blocks,
    # scales that saturate binary16, tiny values with subnormal scales
    say("q4k quantize special values")
    rng = np.random.default_rng(100)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = 0.37
    x[3] = -np.abs(x[3])
    x[4] *= np.float32(3e8)
    x[5] *= np.float32(1e-4)
    x[6, :256] = 0.0
    x[7, ::3] = -0.0
    assert np.array_equal(quantize_gpu(lib, x, 8, 512), orc.q4k_quantize(x))


def test_quantize_then_gemv_matches_dequantised_weights(lib):
    # the quantised matrix feeds q4k_gemv; the product equals the oracle's
    # GEMV on the same bytes (normwise 1e-5)
    rows, cols = 300, 4096
    say("q4k quantize then gemv")
    x = synth.activations(101, rows, cols, outliers=False)
    w = quantize_gpu(lib, x, rows, cols)
    a = synth.activations(102, 2, cols, outliers=True)
    y = empty((2, rows), torch.float32)
    lib.q4k_gemv(dev(w), dev(a), y, 2, rows, cols)
    ref = orc.gemv(w, rows, cols, a)
    err = orc.normalized_max_error(host(y), ref, orc.row_norms(w, rows, cols),
                                   np.linalg.norm(a.astype(np.float64), axis=1))
    assert err <= 1e-5, err
