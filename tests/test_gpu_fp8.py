"""Per-row FP8 (E4M3) recipe on the GPU against the FP8 oracle
("aprender-serve 0.70.2 -- cublas_prefill/fp8_recipe.rs").

Row absmax and the E4M3 codes are compared bit for bit.  The GEMM with the
outer dequant is compared through an envelope around the oracle's exact D.
The bound comes from the arithmetic of gfx950's v_mfma_f32_32x32x64_f8f6f4,
measured with crafted operands (and reproduced exactly, output for output, by
the model below on random and outlier-heavy tiles): within each group of 8
consecutive k the products are aligned to E = the largest exponent sum
e(a) + e(b) of the group and each is truncated toward zero to a multiple of
2^(E - 13); the 64 truncated products of one instruction are summed and added
to the f32 accumulator with one rounding to nearest.  Hence
|D_gpu - D| <= sum_g (n_g - 1) 2^(E_g - 13) + (k/64) u (S + that), with n_g
the products of group g (the one with exponent sum E_g is a multiple of its
grid), S = sum |a_i w_i| and u = 2^-24.  BF16 rounding and the two scalings
are monotone, so every GPU output must lie between the oracle's outputs for
D - bound and D + bound, and most must equal the oracle's output for the
exact D.  At the prefill FFN's full sizes the per-row recipe makes every
sampled (token, weight row) pair self-contained: the oracle quantises only the
sampled rows of x and w."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import fp8_oracle as fp8
from gpu_helpers import dev, empty, host, say

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


def quant_gpu(q4k, x, absmax=None):
    rows, cols = x.shape
    xd = dev(x)
    if absmax is None:
        am = empty((rows,), torch.float32)
        q4k.fp8_absmax_rows(xd, rows, cols, am)
    else:
        am = dev(np.asarray(absmax, np.float32))
    q = empty((rows, cols), torch.uint8)
    q4k.fp8_quantize_rows(xd, rows, cols, am, q)
    return host(q), host(am)


def gemm_gpu(q4k, qa, aa, qw, wa):
    m, k = qa.shape
    n = qw.shape[0]
    y = empty((m, n), torch.float32)
    q4k.fp8_gemm_dequant(dev(qa), dev(aa), dev(qw), dev(wa), y, m, n, k)
    return host(y)


def code_exponent(codes):
    """Unbiased exponent of E4M3 codes (the subnormal and zero codes: -6)."""
    e = (codes.astype(np.int16) >> 3) & 15
    return np.where(e == 0, -6, e - 7).astype(np.int16)


def mfma_bound(qa, qw, chunk_elems=1 << 24):
    """Bound on |D_gpu - D| per output from the matrix instruction's group
    truncation and accumulator rounding (module docstring).  E_g is taken over
    all eight positions of a group, zeros included, which can only widen it."""
    m, k = qa.shape
    n = qw.shape[0]
    kp = (k + 63) // 64 * 64
    ea = np.full((m, kp), -6, np.int16)
    eb = np.full((n, kp), -6, np.int16)
    ea[:, :k] = code_exponent(qa)
    eb[:, :k] = code_exponent(qw)
    nza = np.zeros((m, kp), bool)
    nzb = np.zeros((n, kp), bool)
    nza[:, :k] = (qa & 0x7F) != 0
    nzb[:, :k] = (qw & 0x7F) != 0
    trunc = np.zeros((m, n))
    step = max(1, chunk_elems // max(1, n * kp))
    for t0 in range(0, m, step):
        t1 = min(m, t0 + step)
        es = (ea[t0:t1, None, :] + eb[None, :, :]).reshape(t1 - t0, n, kp // 8, 8)
        cnt = (nza[t0:t1, None, :] & nzb[None, :, :]).reshape(t1 - t0, n, kp // 8, 8).sum(axis=3)
        E = es.max(axis=3).astype(np.float64)
        trunc[t0:t1] = (np.maximum(cnt - 1, 0) * np.exp2(E - 13)).sum(axis=2)
    S = np.abs(fp8.e4m3_decode(qa)) @ np.abs(fp8.e4m3_decode(qw)).T
    return trunc + (kp // 64) * U32 * (S + trunc) * 1.0001


def check_envelope(y, qa, aa, qw, wa, min_equal=0.9):
    """y within the oracle's outputs for D -+ mfma_bound, and at least
    `min_equal` of it equal to the oracle's output for the exact D."""
    D = fp8.gemm_codes(qa, qw)
    err = mfma_bound(qa, qw)
    lo = fp8.dequant_outer(D - err, aa, wa)
    hi = fp8.dequant_outer(D + err, aa, wa)
    ref = fp8.dequant_outer(D, aa, wa)
    assert np.all(np.isfinite(y))
    bad = ~((lo <= y) & (y <= hi))
    assert not np.any(bad), f"{int(bad.sum())} outputs outside the envelope, first at {np.argwhere(bad)[0]}"
    equal = float(np.mean(y == ref))
    assert equal >= min_equal, f"only {equal:.4f} of the outputs equal the oracle's"
    return equal


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (7, 100), (4, 16), (33, 4096), (2, 5120),
                                       (5, 17408), (300, 48)])
def test_absmax_and_codes_bit_exact(lib, rows, cols):
    say(f"fp8 quantize rows={rows} cols={cols}")
    x, _ = synth.fp8_case(rows, 1, cols, sub=rows * 7 + cols)
    x[rows // 2] = 0.0                     # an all-zero row: absmax 0, scale 448
    if cols > 2:
        x[0, 1] = -0.0
    q, am = quant_gpu(lib, x)
    q_ref, am_ref = fp8.quantize_rows(x)
    assert np.array_equal(am.view(np.uint32), am_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def e4m3_grid_values():
    """Every positive finite E4M3 value, every midpoint between neighbours
    (the ties), values just either side of each midpoint, and magnitudes past
    448 (saturation), with both signs."""
    vals = np.sort(fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    f32 = lambda v: np.asarray(v, np.float32)
    near = np.concatenate([np.nextafter(f32(mids), f32(0)), np.nextafter(f32(mids), f32(np.inf))])
    big = f32([448.0, 449.0, 463.99, 464.0, 464.01, 480.0, 1e6, 3e38])
    pos = np.concatenate([f32(vals), f32(mids), near, big])
    return np.concatenate([pos, -pos]).astype(np.float32)


@pytest.mark.parametrize("pad_to", [16, 1])
def test_codes_on_the_e4m3_grid(lib, pad_to):
    # absmax 448 makes the scale exactly 1, so the encoder sees the values as given
    v = e4m3_grid_values()
    cols = (len(v) + pad_to - 1) // pad_to * pad_to + (0 if pad_to > 1 else 1)
    x = np.zeros((2, cols), np.float32)
    x[0, :len(v)] = v
    x[1, :len(v)] = v[::-1] * np.float32(2.0 ** -3)
    absmax = np.array([448.0, 448.0], np.float32)
    say(f"fp8 quantize grid cols={cols}")
    q, _ = quant_gpu(lib, x, absmax)
    q_ref, _ = fp8.quantize_rows(x, absmax)
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (5, 37, 48), (130, 200, 272), (300, 384, 1024),
                                   (64, 128, 5120), (257, 129, 4096 + 16), (513, 16384 + 40, 64)])
def test_gemm_dequant_envelope(lib, m, n, k):
    # the last shape's outputs are checked on every 7th weight row and the
    # ragged last tile
    say(f"fp8 gemm m={m} n={n} k={k}")
    x, w = synth.fp8_case(m, n, k, sub=m + n + k)
    qa, aa = fp8.quantize_rows(x)
    qw, wa = fp8.quantize_rows(w)
    y = gemm_gpu(lib, qa, aa, qw, wa)
    rows = np.unique(np.concatenate([np.arange(0, n, 7), np.arange(max(0, n - 40), n)])) if n > 4096 \
        else np.arange(n)
    equal = check_envelope(y[:, rows], qa, aa, qw[rows], wa[rows])
    say(f"  {equal:.5f} of the outputs equal the oracle's")


def test_gemm_maximum_k(lib):
    # k = 2^20, the largest the entry point takes: 8192 stages of 128
    m, n, k = 3, 5, 1 << 20
    say(f"fp8 gemm maximum k m={m} n={n} k={k}")
    x, w = synth.fp8_case(m, n, k, sub=77)
    qa, aa = fp8.quantize_rows(x)
    qw, wa = fp8.quantize_rows(w)
    y = gemm_gpu(lib, qa, aa, qw, wa)
    check_envelope(y, qa, aa, qw, wa, min_equal=0.0)


def test_gemm_zero_rows_and_saturated_codes(lib):
    # all-zero token and weight rows (absmax 0, taken as 1), and rows of 448s:
    # |D| up to 448^2 k stays far inside the f32 and BF16 exponent range
    m, n, k = 70, 140, 512
    x, w = synth.fp8_case(m, n, k, sub=11)
    x[3] = 0.0
    w[5] = 0.0
    x[9] = 1.0
    w[7] = -3.0
    qa, aa = fp8.quantize_rows(x)
    qw, wa = fp8.quantize_rows(w)
    assert np.all(qa[9] == 0x7E) and np.all(qw[7] == 0xFE)
    y = gemm_gpu(lib, qa, aa, qw, wa)
    assert np.all(y[3] == 0) and np.all(y[:, 5] == 0)
    check_envelope(y, qa, aa, qw, wa)
    # the saturated pair: D = -448^2 k exactly (and in BF16), so Y is -3 k up
    # to the two rounded factors 1/448 and 3/448
    assert abs(y[9, 7] / (-3.0 * k) - 1) <= 4 * U32


def sample_rows(count, tile, per_tile):
    """`per_tile` rows of every `tile`-row tile, at positions that differ from
    tile to tile, and the last row."""
    rows = []
    for i in range((count + tile - 1) // tile):
        for j in range(per_tile):
            rows.append(min(count - 1, tile * i + (37 * i + 53 * j + 5) % tile))
    return np.array(sorted(set(rows + [count - 1])))


@pytest.mark.parametrize("m,n,k", [(512, 17408, 5120), (512, 5120, 17408), (2048, 17408, 5120),
                                   (2048, 5120, 17408)])
def test_recipe_full_size_sampled(lib, m, n, k):
    """The whole recipe on the GPU at the prefill FFN's sizes (quantise x and w,
    GEMM with the outer dequant), in the launch configuration the benchmark
    times; sampled rows checked against the oracle from the f32 inputs."""
    toks = sample_rows(m, 256, 3)
    chans = sample_rows(n, 128, 2)
    say(f"fp8 recipe full size m={m} n={n} k={k} ({len(toks)} tokens x {len(chans)} rows)")
    x, w = synth.fp8_case(m, n, k, sub=1000 + m + n)
    xd, wd = dev(x), dev(w)
    am, wam = empty((m,), torch.float32), empty((n,), torch.float32)
    qa, qw = empty((m, k), torch.uint8), empty((n, k), torch.uint8)
    y = empty((m, n), torch.float32)
    lib.fp8_absmax_rows(wd, n, k, wam)
    lib.fp8_quantize_rows(wd, n, k, wam, qw)
    lib.fp8_absmax_rows(xd, m, k, am)
    lib.fp8_quantize_rows(xd, m, k, am, qa)
    lib.fp8_gemm_dequant(qa, am, qw, wam, y, m, n, k)
    ti, ci = torch.as_tensor(toks, device="cuda"), torch.as_tensor(chans, device="cuda")
    y_s = host(y.index_select(0, ti).index_select(1, ci))
    qa_s, qw_s = host(qa.index_select(0, ti)), host(qw.index_select(0, ci))
    del xd, wd, qa, qw, y
    qa_ref, aa_ref = fp8.quantize_rows(x[toks])
    qw_ref, wa_ref = fp8.quantize_rows(w[chans])
    assert np.array_equal(qa_s, qa_ref) and np.array_equal(qw_s, qw_ref)
    equal = check_envelope(y_s, qa_ref, aa_ref, qw_ref, wa_ref)
    say(f"  {equal:.5f} of the sampled outputs equal the oracle's")
