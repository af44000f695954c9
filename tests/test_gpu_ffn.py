"""End-to-end SwiGLU FFN on the GPU: relative L2 <= 2e-3 against the oracle."""
import numpy as np
import pytest
import torch

import gemm_block_q4_amd as q4kmod
from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say, workspace

pytestmark = pytest.mark.gpu
TOL = 2e-3


def ffn_gpu(q4k, wg, wu, wd, x, hidden, inter, regime=0, bf16=False):
    m = x.shape[0]
    y = empty((m, hidden), torch.float32)
    ws = workspace(q4k, m, hidden, inter, 0, regime)
    xin = dev(synth.to_bf16_bits(x).view(np.int16)) if bf16 else dev(x)
    q4k.ffn_swiglu_q4k(dev(wg), dev(wu), dev(wd), xin, q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32,
                       m, hidden, inter, y, ws, regime=regime)
    return host(y)


def test_tiny_ffn(lib):
    say("ffn tiny 256/768 m=1")
    wg, wu, wd = synth.dense_ffn_weights(synth.TINY_FFN, 256, 768)
    x = synth.activations(synth.TINY_FFN, 1, 256, outliers=False)
    y = ffn_gpu(lib, wg, wu, wd, x, 256, 768)
    assert orc.relative_l2(y, orc.ffn_decode(wg, wu, wd, 256, 768, x)) <= TOL


@pytest.fixture(scope="module")
def decode7b():
    return synth.dense_ffn_weights(synth.DECODE_FFN_7B, 4096, 11008)


@pytest.mark.parametrize("m", [1, 4, 8])
def test_decode_ffn_7b(lib, decode7b, m):
    say(f"ffn decode 4096/11008 m={m}")
    wg, wu, wd = decode7b
    x = synth.activations(synth.DECODE_FFN_7B, m, 4096, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, 4096, 11008)
    ref = orc.ffn_decode(wg, wu, wd, 4096, 11008, x)
    assert orc.relative_l2(y, ref) <= TOL


@pytest.mark.parametrize("m,regime", [(9, 0), (65, 0), (130, 0), (3, 2), (1, 2)])
def test_prefill_ffn_small(lib, m, regime):
    say(f"ffn prefill 512/768 m={m} regime={regime}")
    hidden, inter = 512, 768
    wg, wu, wd = synth.dense_ffn_weights(90, hidden, inter)
    x = synth.activations(90, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, regime=regime, bf16=True)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    ref = orc.ffn_prefill(wg, wu, wd, hidden, inter, xb)
    assert orc.relative_l2(y, ref) <= TOL


@pytest.mark.parametrize("m,hidden,inter", [(300, 256, 2048), (130, 512, 1536), (200, 512, 768)])
def test_prefill_ffn_k_split(lib, m, hidden, inter):
    # inter >= 2 * hidden leaves room for the down pass's k-split partials
    # (8 and 3 splits here); 512/768 has none and runs unsplit
    say(f"ffn prefill k-split {hidden}/{inter} m={m}")
    wg, wu, wd = synth.dense_ffn_weights(91, hidden, inter)
    x = synth.activations(91, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, regime=2, bf16=True)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    ref = orc.ffn_prefill(wg, wu, wd, hidden, inter, xb)
    assert orc.relative_l2(y, ref) <= TOL


@pytest.mark.parametrize("m,hidden,inter", [(1, 512, 768), (3, 512, 768), (6, 4608, 512)])
def test_decode_ffn_bf16_input(lib, m, hidden, inter):
    # bf16 activations through the one-token and the matrix-core GEMVs
    say(f"ffn decode bf16 x m={m} {hidden}/{inter}")
    wg, wu, wd = synth.dense_ffn_weights(93, hidden, inter)
    x = synth.activations(93, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, regime=1, bf16=True)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    assert orc.relative_l2(y, orc.ffn_decode(wg, wu, wd, hidden, inter, xb)) <= TOL


def test_decode_regime_forced_m8_matches(lib):
    say("ffn decode regime forced, m=8, 512/768")
    hidden, inter = 512, 768
    wg, wu, wd = synth.dense_ffn_weights(91, hidden, inter)
    x = synth.activations(91, 8, hidden, outliers=True)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, regime=1)
    assert orc.relative_l2(y, orc.ffn_decode(wg, wu, wd, hidden, inter, x)) <= TOL


@pytest.mark.parametrize("m", [1, 3])
def test_decode_ffn_wide_inter(lib, m):
    # inter 18432 > 16384: the down pass's one-token rows span five wavefronts
    # with four activation units per thread and LDS above 64 KiB
    hidden, inter = 512, 18432
    say(f"ffn decode wide inter {hidden}/{inter} m={m}")
    wg, wu, wd = synth.dense_ffn_weights(95, hidden, inter)
    x = synth.activations(95, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter)
    assert orc.relative_l2(y, orc.ffn_decode(wg, wu, wd, hidden, inter, x)) <= TOL


@pytest.mark.parametrize("m,hidden,inter", [(2, 1024, 4096), (5, 2560, 8192), (8, 2560, 8192), (8, 768, 4352)])
def test_decode_ffn_split_down(lib, m, hidden, inter):
    # 2..8 tokens with the down pass's k split in two halves that add into y
    # (zeroed by the gate/up pass): one or two row tiles per workgroup, an odd
    # block count (17 = 8 + 9).  y starts as NaN, and a second call with other
    # activations must not accumulate onto the first call's result.
    say(f"ffn decode split down {hidden}/{inter} m={m}")
    wg, wu, wd = synth.dense_ffn_weights(96, hidden, inter)
    ws = workspace(lib, m, hidden, inter)
    gw, uw, dw = dev(wg), dev(wu), dev(wd)
    y = empty((m, hidden), torch.float32)
    y.fill_(float("nan"))
    for sub in (m, m + 100):
        x = synth.activations(96, m, hidden, outliers=True, sub=sub)
        lib.ffn_swiglu_q4k(gw, uw, dw, dev(x), lib.Q4K_F32, m, hidden, inter, y, ws)
        assert orc.relative_l2(host(y), orc.ffn_decode(wg, wu, wd, hidden, inter, x)) <= TOL


def _scale_rows(w, rows, k, factor):
    """Multiply d and dmin of every block of the given rows by a power of two."""
    blk = w.reshape(-1, k // 256, 144)
    for r in rows:
        for off in (0, 2):
            h = blk[r, :, off:off + 2].copy().view(np.float16)
            blk[r, :, off:off + 2] = (h.astype(np.float32) * factor).astype(np.float16).view(np.uint8)


def test_decode_ffn_split_uneven_magnitudes(lib):
    # h with uneven magnitudes on the split down pass, whose activation scale
    # is per (token, chunk of 512 values): all-zero rows (gate rows 0..31
    # without scale), 16 rows 2^12 above the rest of their chunk (up rows
    # 64..79), 16 rows 2^-10 below (up rows 1024..1039), and a token whose x
    # and hence h are all zero (y exactly zero)
    m, hidden, inter = 3, 1024, 4096
    say("ffn decode split down, uneven magnitudes 1024/4096 m=3")
    wg, wu, wd = synth.dense_ffn_weights(98, hidden, inter)
    _scale_rows(wg, range(0, 32), hidden, 0.0)
    _scale_rows(wu, range(64, 80), hidden, 2.0 ** 12)
    _scale_rows(wu, range(1024, 1040), hidden, 2.0 ** -10)
    x = synth.activations(98, m, hidden, outliers=True)
    x[1] = 0.0
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter)
    ref = orc.ffn_decode(wg, wu, wd, hidden, inter, x)
    assert np.all(y[1] == 0.0)
    for t in (0, 2):
        assert orc.relative_l2(y[t], ref[t]) <= TOL


def test_decode_ffn_in_place(lib):
    # y aliasing x: the down pass runs unsplit, so x is intact while the
    # gate/up pass reads it
    m, hidden, inter = 4, 1024, 4096
    say("ffn decode in place 1024/4096 m=4")
    wg, wu, wd = synth.dense_ffn_weights(97, hidden, inter)
    x = synth.activations(97, m, hidden, outliers=True)
    buf = dev(x)
    lib.ffn_swiglu_q4k(dev(wg), dev(wu), dev(wd), buf, lib.Q4K_F32, m, hidden, inter, buf,
                       workspace(lib, m, hidden, inter))
    assert orc.relative_l2(host(buf), orc.ffn_decode(wg, wu, wd, hidden, inter, x)) <= TOL


@pytest.mark.parametrize("m", [1, 4, 8])
def test_decode_q8_ffn_7b(lib, decode7b, m):
    # Q8_1 decode regime: the prefill arithmetic (Q8_1 of x and of h) on the
    # integer-dot GEMVs
    say(f"ffn decode_q8 4096/11008 m={m}")
    wg, wu, wd = decode7b
    x = synth.activations(synth.DECODE_FFN_7B, m, 4096, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, 4096, 11008, regime=q4kmod.Q4K_REGIME_DECODE_Q8)
    assert orc.relative_l2(y, orc.ffn_prefill(wg, wu, wd, 4096, 11008, x)) <= TOL


@pytest.mark.parametrize("m,hidden,inter,bf16", [
    (2, 512, 768, True), (3, 4608, 512, False),   # gate/up rows span two wavefronts
    (5, 512, 8448, True),                          # down rows span three
    (7, 256, 256, False), (1, 8192, 1024, True), (6, 1024, 2816, False)])
def test_decode_q8_ffn_shapes(lib, m, hidden, inter, bf16):
    say(f"ffn decode_q8 {hidden}/{inter} m={m} bf16={bf16}")
    wg, wu, wd = synth.dense_ffn_weights(94, hidden, inter)
    x = synth.activations(94, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, regime=q4kmod.Q4K_REGIME_DECODE_Q8, bf16=bf16)
    xr = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) if bf16 else x
    assert orc.relative_l2(y, orc.ffn_prefill(wg, wu, wd, hidden, inter, xr)) <= TOL
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("m,hidden", [(130, 512), (300, 1024), (130, 1280)])
def test_prefill_ffn_gate_up_tail_split(lib, m, hidden):
    # 272 row tiles of the fused gate/up pass x 2 or 3 token tiles leave a
    # partial last round on 256 compute units: the last 16 row tiles run as a
    # k-split pass (2, 4 and 3 splits: 5 blocks of k cannot go into 4
    # non-empty splits; the last token tile ragged) whose gate and
    # up sums are added by the finishing kernel; every fifth token (every
    # lane position of a token tile over the sample) and the last are compared
    inter = 17408
    tokens = sorted(set(range(0, m, 5)) | {m - 1})
    say(f"ffn prefill gate/up tail split {hidden}/{inter} m={m}")
    wg, wu, wd = synth.dense_ffn_weights(92, hidden, inter)
    x = synth.activations(92, m, hidden, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, hidden, inter, bf16=True)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    ref = orc.ffn_prefill(wg, wu, wd, hidden, inter, xb, tokens=tokens)
    assert orc.relative_l2(y[tokens], ref) <= TOL


@pytest.fixture(scope="module")
def prefill_weights():
    return synth.dense_ffn_weights(synth.PREFILL_FFN, 5120, 17408)


def tile_sample(m, tile=128):
    """One token from every tile of `tile` tokens (a different position in each
    tile, so that different lanes and accumulator rows are compared) plus the
    last token."""
    tokens = [min(m - 1, tile * i + (37 * i + 5) % tile) for i in range((m + tile - 1) // tile)]
    return sorted(set(tokens + [m - 1]))


@pytest.mark.parametrize("m", [512, 2048])
def test_prefill_ffn_full_size(lib, prefill_weights, m):
    tokens = tile_sample(m)
    say(f"ffn prefill 5120/17408 m={m} (sampled tokens {tokens})")
    wg, wu, wd = prefill_weights
    x = synth.activations(synth.PREFILL_FFN, m, 5120, outliers=True, sub=m)
    y = ffn_gpu(lib, wg, wu, wd, x, 5120, 17408, bf16=True)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    ref = orc.ffn_prefill(wg, wu, wd, 5120, 17408, xb, tokens=tokens)
    assert orc.relative_l2(y[tokens], ref) <= TOL
    assert np.all(np.isfinite(y))


def moe_gpu(q4k, banks, x, ids, wts, n_exp, hidden, inter, bf16=False):
    m, top_k = ids.shape
    y = empty((m, hidden), torch.float32)
    ws = workspace(q4k, m, hidden, inter, top_k, 0)
    bg, bu, bd = banks
    xin = dev(synth.to_bf16_bits(x).view(np.int16)) if bf16 else dev(x)
    q4k.ffn_swiglu_q4k(dev(bg), dev(bu), dev(bd), xin, q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32, m,
                       hidden, inter, y, ws, n_experts=n_exp, ids=dev(ids), wts=dev(wts),
                       top_k=top_k)
    return host(y)


def test_moe_decode_config(lib):
    say("moe 64 experts top-8, 4 tokens, 2048/768")
    n_exp, hidden, inter, m, k = 64, 2048, 768, 4, 8
    banks = synth.moe_banks(synth.MOE_DECODE, n_exp, hidden, inter)
    x = synth.activations(synth.MOE_DECODE, m, hidden, outliers=False)
    ids, wts = synth.router(synth.MOE_DECODE, m, n_exp, k)
    y = moe_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter)
    ref = orc.moe_decode(*banks, n_exp, hidden, inter, x, ids, wts)
    assert orc.relative_l2(y, ref) <= TOL


def test_moe_duplicates_and_out_of_range_ids(lib):
    say("moe duplicate and out-of-range ids")
    n_exp, hidden, inter, m, k = 5, 256, 512, 3, 4
    banks = synth.moe_banks(92, n_exp, hidden, inter)
    x = synth.activations(92, m, hidden, outliers=True)
    ids = np.array([[1, 1, 4, 9], [0, 2, -1, 2], [3, 3, 3, 3]], dtype=np.int32)
    wts = np.array([[0.5, 0.25, 0.125, 2.0], [1.0, 0.5, 3.0, -1.0], [0.1, 0.2, 0.3, 0.4]],
                   dtype=np.float32)
    y = moe_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter)
    valid = (ids >= 0) & (ids < n_exp)
    ref = orc.moe_decode(*banks, n_exp, hidden, inter, x, np.where(valid, ids, 0),
                         np.where(valid, wts, 0).astype(np.float32))
    assert orc.relative_l2(y, ref) <= TOL


@pytest.mark.parametrize("inter", [3072, 4096])
def test_moe_top8_wide_down(lib, inter):
    # top-8 with down rows of 48 or 64 slices: the fused down pass holds eight
    # wavefronts' digits and the slot results in more than 64 KiB of LDS
    n_exp, hidden, m, k = 10, 512, 3, 8
    say(f"moe top-8 {hidden}/{inter}")
    banks = synth.moe_banks(96, n_exp, hidden, inter)
    x = synth.activations(96, m, hidden, outliers=True)
    ids, wts = synth.router(96, m, n_exp, k)
    y = moe_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter)
    ref = orc.moe_decode(*banks, n_exp, hidden, inter, x, ids, wts)
    assert orc.relative_l2(y, ref) <= TOL


@pytest.mark.parametrize("hidden,inter,bf16", [(4608, 512, False), (512, 4608, True)])
def test_moe_wide_rows(lib, hidden, inter, bf16):
    # rows that span wavefronts in the gate/up pass (hidden 4608) or the down
    # pass (inter 4608); bf16 activations
    say(f"moe wide rows {hidden}/{inter} bf16={bf16}")
    n_exp, m, k = 3, 2, 2
    banks = synth.moe_banks(94, n_exp, hidden, inter)
    x = synth.activations(94, m, hidden, outliers=True)
    ids = np.array([[2, 0], [0, 1]], dtype=np.int32)
    wts = np.array([[0.75, 0.25], [0.5, 1.5]], dtype=np.float32)
    y = moe_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter, bf16=bf16)
    xr = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) if bf16 else x
    ref = orc.moe_decode(*banks, n_exp, hidden, inter, xr, ids, wts)
    assert orc.relative_l2(y, ref) <= TOL
