"""Pins of the oracle's Q4_K weight quantiser (load-time encoding).

Checked against facts the format fixes rather than against the quantiser's own
formulas: the quant packing is the inverse of the (separately pinned) unpack,
blocks whose values a Q4_K block represents exactly come back bit for bit,
degenerate blocks, and a reconstruction bound that follows from the block
grid (each value within half a step of its grid point, plus the 6-bit
rounding of the sub-block scale and min)."""
import numpy as np
import pytest

from oracle import q4k_oracle as orc


def test_pack_quants_is_the_inverse_of_unpack():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, (50, 256)).astype(np.uint8)
    assert np.array_equal(orc.unpack_quants(orc.pack_quants(q)), q)
    b = rng.integers(0, 256, (50, 128), dtype=np.uint8)
    assert np.array_equal(orc.pack_quants(orc.unpack_quants(b)), b)


def representable_blocks(rng, nblk):
    """Blocks whose 6-bit maxima are 63 and whose sub-blocks span q = 0..15:
    exactly the values the fit maps back to the same fields."""
    blocks = np.zeros((nblk, 144), dtype=np.uint8)
    d = rng.uniform(1e-3, 1e-2, nblk).astype(np.float32).astype(np.float16)
    dmin = rng.uniform(1e-3, 1e-2, nblk).astype(np.float32).astype(np.float16)
    sc = rng.integers(1, 64, (nblk, 8))
    mn = rng.integers(0, 64, (nblk, 8))
    sc[np.arange(nblk), rng.integers(0, 8, nblk)] = 63
    mn[np.arange(nblk), rng.integers(0, 8, nblk)] = 63
    q = rng.integers(0, 16, (nblk, 8, 32))
    for j in range(8):
        i0, i15 = rng.choice(32, 2, replace=False)
        q[:, j, i0] = 0
        q[:, j, i15] = 15
    blocks[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nblk, 2)
    blocks[:, 4:16] = orc.pack_scale_min(sc, mn)
    blocks[:, 16:] = orc.pack_quants(q.reshape(nblk, 256).astype(np.uint8))
    return blocks


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_representable_blocks_round_trip_bit_exact(seed):
    rng = np.random.default_rng(seed)
    rows, nb = 6, 5
    blocks = representable_blocks(rng, rows * nb)
    w = blocks.reshape(-1)
    x = orc.dequantize(w, rows, nb * 256).astype(np.float32)
    assert np.array_equal(orc.q4k_quantize(x), w)


def test_zero_and_constant_blocks():
    assert not np.any(orc.q4k_quantize(np.zeros((2, 512), np.float32)))
    # no negative value: the stored min is +0 (bytes 2-3 zero), not -0
    assert not np.any(orc.q4k_quantize(np.full((1, 256), 0.37, np.float32))[2:4])
    # (binary16 d: below about 6.1e-5 * 15 * 63 = 0.058 the scale is subnormal
    # and loses bits; much smaller constants underflow it)
    for c in (0.37, 3.0e3, 12.0):
        x = np.full((1, 256), c, np.float32)
        r = orc.dequantize(orc.q4k_quantize(x), 1, 256)
        assert np.all(np.abs(r - c) <= c * 2.0 ** -10), (c, r[0, :4])
    x = np.full((1, 256), -0.8, np.float32)       # all negative: the min carries it
    r = orc.dequantize(orc.q4k_quantize(x), 1, 256)
    assert np.all(np.abs(r + 0.8) <= 0.8 * 2.0 ** -10)


@pytest.mark.parametrize("outliers", [False, True])
def test_reconstruction_within_grid_bound(outliers):
    from gemm_block_q4_amd import synth
    rows, cols = 8, 2048
    x = synth.activations(7, rows, cols, outliers=outliers)
    w = orc.q4k_quantize(x)
    d, dmin, sc, mn, _ = orc.block_fields(w, rows, cols)
    r = orc.dequantize(w, rows, cols)
    ds = np.repeat((d[..., None] * sc).reshape(rows, -1), 32, axis=1)
    dm = np.repeat((dmin[..., None] * mn).reshape(rows, -1), 32, axis=1)
    dd = np.repeat(d, 256, axis=1)
    dmn = np.repeat(dmin, 256, axis=1)
    xx = x.astype(np.float64)
    bound = ds / 2 + 7.5 * dd + 0.5 * dmn + 1e-3 * (np.abs(xx) + 16 * ds + dm)
    assert np.all(np.abs(r - xx) <= bound)
    # and the fit is not trivially loose: mean error well below a step
    assert np.mean(np.abs(r - xx)) < np.mean(ds) / 2


def test_rejects_bad_shapes_and_non_finite():
    with pytest.raises(ValueError):
        orc.q4k_quantize(np.zeros((1, 300), np.float32))
    with pytest.raises(ValueError):
        orc.q4k_quantize(np.full((1, 256), np.inf, np.float32))
