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


def tie_inputs(rows, cols, seed):
    """Weights at the half-integer points of their own block grid.

    Each 32-value sub-block gets its minimum -L_j (0 for half of them) at
    position 0 and its maximum 15 S - L_j at position 1, with one step S per
    block, so the oracle's fit gives every sub-block the same scale code and
    the quantiser keeps that fit however the other 30 values move inside
    [-L_j, 15 S - L_j].  Those are then set to binary32 (k + 1/2) ds - dm for
    the block's stored ds = d sc_j and dm = dmin m_j: (x + dm) / ds is at or
    within a few units of the last place of k + 1/2, where the rounding of
    the quotient and then to an integer decides the code."""
    rng = np.random.default_rng(seed)
    nb = cols // 256
    x = np.zeros((rows, nb, 8, 32), dtype=np.float32)
    S = rng.uniform(0.01, 2.0, (rows, nb, 1)).astype(np.float32)
    L = np.where(rng.random((rows, nb, 8)) < 0.5, 0.0, rng.uniform(0.1, 5.0, (rows, nb, 8))).astype(np.float32)
    x[..., 0] = -L
    x[..., 1] = (np.float32(15.0) * S - L).astype(np.float32)
    x[..., 2:] = (rng.uniform(0, 15, (rows, nb, 8, 30)) * S[..., None] - L[..., None]).astype(np.float32)
    x = x.reshape(rows, cols)
    d, dmin, sc, mn, _ = orc.block_fields(orc.q4k_quantize(x), rows, cols)
    ds = (d.astype(np.float32)[..., None] * sc.astype(np.float32)).astype(np.float32)
    dm = (dmin.astype(np.float32)[..., None] * mn.astype(np.float32)).astype(np.float32)
    k = rng.integers(0, 15, (rows, nb, 8, 30)).astype(np.float32)
    xb = x.reshape(rows, nb, 8, 32)
    xb[..., 2:] = ((k + np.float32(0.5)) * ds[..., None] - dm[..., None]).astype(np.float32)
    xb[..., 2:] = np.clip(xb[..., 2:], xb[..., :1], xb[..., 1:2])  # stay inside the fitted range
    out = xb.reshape(rows, cols)
    # the fit is unchanged by the move
    assert np.array_equal(orc.block_fields(orc.q4k_quantize(out), rows, cols)[2], sc)
    return out


@pytest.mark.parametrize("rows,cols", [(64, 1024), (37, 2304)])
def test_quantize_grid_midpoints_bit_exact(lib, rows, cols):
    # quotients at or next to k + 1/2: the rounding of the division and then
    # to an integer (ties to even) must match the oracle's binary32 steps
    say(f"q4k quantize grid midpoints rows={rows} cols={cols}")
    x = tie_inputs(rows, cols, 103 + rows)
    ref = orc.q4k_quantize(x)
    assert np.array_equal(quantize_gpu(lib, x, rows, cols), ref)


@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_full_size_bit_exact(lib, bf16):
    # the [11008, 4096] matrix bench.py times, every byte against the oracle
    rows, cols = 11008, 4096
    say(f"q4k quantize full size {rows}x{cols} bf16={bf16}")
    x = synth.activations(synth.GEMV_SWEEP, rows, cols, False, sub=200)
    if bf16:
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    assert np.array_equal(quantize_gpu(lib, x, rows, cols, bf16=bf16), orc.q4k_quantize(x))
