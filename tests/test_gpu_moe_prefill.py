"""Top-k MoE FFN in the prefill regime (the grouped MMQ passes) against the
oracle at the prefill quantisation points: relative L2 <= 2e-3, as for the
dense FFN.  Covers the routed-MoE workload at 64..512 tokens, experts with
several 128-row tiles and with none, out-of-range ids and bf16 input."""
import numpy as np
import pytest
import torch

from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say, workspace

pytestmark = pytest.mark.gpu
TOL = 2e-3


def moe_prefill_gpu(q4k, banks, x, ids, wts, n_exp, hidden, inter, bf16=False, regime=0):
    m, top_k = ids.shape
    y = empty((m, hidden), torch.float32)
    ws = workspace(q4k, m, hidden, inter, top_k, regime)
    bg, bu, bd = banks
    xin = dev(synth.to_bf16_bits(x).view(np.int16)) if bf16 else dev(x)
    q4k.ffn_swiglu_q4k(dev(bg), dev(bu), dev(bd), xin, q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32, m,
                       hidden, inter, y, ws, n_experts=n_exp, ids=dev(ids), wts=dev(wts),
                       top_k=top_k, regime=regime)
    return host(y)


def sample_tokens(m, tile=64):
    """One token from every `tile` tokens, at positions that vary, and the last."""
    toks = [min(m - 1, tile * i + (29 * i + 7) % tile) for i in range((m + tile - 1) // tile)]
    return sorted(set(toks + [m - 1]))


@pytest.fixture(scope="module")
def moe_config_banks():
    return synth.moe_banks(synth.MOE_DECODE, 64, 2048, 768)


@pytest.mark.parametrize("m", [64, 200, 512, 2048])
def test_moe_prefill_routed_config(lib, moe_config_banks, m):
    # the routed-MoE workload's experts and router (64 experts, top-8,
    # 2048/768) at prefill token counts
    n_exp, hidden, inter, k = 64, 2048, 768, 8
    tokens = sample_tokens(m)
    say(f"moe prefill 64 experts top-8 2048/768 m={m} (sampled tokens {tokens})")
    x = synth.activations(synth.MOE_DECODE, m, hidden, outliers=True, sub=m)
    ids, wts = synth.router(synth.MOE_DECODE, m, n_exp, k, seed=m)
    y = moe_prefill_gpu(lib, moe_config_banks, x, ids, wts, n_exp, hidden, inter)
    ref = orc.moe_prefill(*moe_config_banks, n_exp, hidden, inter, x, ids, wts, tokens=tokens)
    assert np.all(np.isfinite(y))
    assert orc.relative_l2(y[tokens], ref) <= TOL


@pytest.mark.parametrize("m,k,n_exp,bf16", [(300, 2, 2, False), (9, 3, 7, True), (40, 1, 3, False)])
def test_moe_prefill_tiles_per_expert(lib, m, k, n_exp, bf16):
    # 2 experts x 300 tokens x top-2: every expert takes 300 rows, three tiles
    # (the last ragged); 9 tokens: the smallest automatic prefill call; top-1
    hidden, inter = 512, 768
    say(f"moe prefill tiles m={m} top-{k} experts={n_exp} bf16={bf16}")
    banks = synth.moe_banks(97, n_exp, hidden, inter)
    x = synth.activations(97, m, hidden, outliers=True, sub=m)
    ids, wts = synth.router(97, m, n_exp, k, seed=m)
    y = moe_prefill_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter, bf16=bf16)
    xr = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) if bf16 else x
    ref = orc.moe_prefill(*banks, n_exp, hidden, inter, xr, ids, wts)
    assert orc.relative_l2(y, ref) <= TOL


def test_moe_prefill_out_of_range_ids_and_idle_experts(lib):
    # ids outside [0, n_exp) contribute nothing; experts 5..9 get no pair;
    # the prefill regime forced at 4 tokens
    n_exp, hidden, inter, m, k = 10, 256, 512, 4, 4
    say("moe prefill out-of-range ids, idle experts")
    banks = synth.moe_banks(98, n_exp, hidden, inter)
    x = synth.activations(98, m, hidden, outliers=True)
    ids = np.array([[1, 1, 4, 10], [0, 2, -1, 2], [3, 3, 3, 3], [-7, 4, 0, 1]], dtype=np.int32)
    wts = np.array([[0.5, 0.25, 0.125, 2.0], [1.0, 0.5, 3.0, -1.0], [0.1, 0.2, 0.3, 0.4],
                    [5.0, 0.7, 0.2, 0.1]], dtype=np.float32)
    y = moe_prefill_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter, regime=2)
    valid = (ids >= 0) & (ids < n_exp)
    ref = orc.moe_prefill(*banks, n_exp, hidden, inter, x, np.where(valid, ids, 0),
                          np.where(valid, wts, 0).astype(np.float32))
    assert orc.relative_l2(y, ref) <= TOL


def test_moe_prefill_two_calls_reuse_the_workspace(lib):
    # a second call with other routing on the same workspace (the tile table
    # and pair list are rebuilt on the GPU each call)
    n_exp, hidden, inter, m, k = 6, 256, 256, 33, 2
    say("moe prefill two calls")
    banks = synth.moe_banks(99, n_exp, hidden, inter)
    ws = workspace(lib, m, hidden, inter, k, 0)
    bg, bu, bd = (dev(b) for b in banks)
    for seed in (1, 2):
        x = synth.activations(99, m, hidden, outliers=False, sub=seed)
        ids, wts = synth.router(99, m, n_exp, k, seed=seed)
        y = empty((m, hidden), torch.float32)
        lib.ffn_swiglu_q4k(bg, bu, bd, dev(x), lib.Q4K_F32, m, hidden, inter, y, ws, n_experts=n_exp,
                           ids=dev(ids), wts=dev(wts), top_k=k)
        ref = orc.moe_prefill(*banks, n_exp, hidden, inter, x, ids, wts)
        assert orc.relative_l2(host(y), ref) <= TOL


def test_moe_prefill_many_experts(lib):
    # 300 experts (several per lane of the routing scan), top-4, most of them
    # idle; pairs of one token on distinct experts
    n_exp, hidden, inter, m, k = 300, 256, 256, 24, 4
    say("moe prefill 300 experts top-4")
    banks = synth.moe_banks(95, n_exp, hidden, inter)
    x = synth.activations(95, m, hidden, outliers=True)
    ids, wts = synth.router(95, m, n_exp, k)
    y = moe_prefill_gpu(lib, banks, x, ids, wts, n_exp, hidden, inter)
    ref = orc.moe_prefill(*banks, n_exp, hidden, inter, x, ids, wts)
    assert orc.relative_l2(y, ref) <= TOL


def test_moe_prefill_output_not_16_byte_aligned(lib):
    # y one float past a 16-byte boundary: the combine takes its
    # one-column-per-thread form
    n_exp, hidden, inter, m, k = 5, 256, 256, 20, 2
    say("moe prefill, y offset by one float")
    banks = synth.moe_banks(94, n_exp, hidden, inter)
    x = synth.activations(94, m, hidden, outliers=True)
    ids, wts = synth.router(94, m, n_exp, k)
    buf = empty((m * hidden + 1,), torch.float32)
    y = buf[1:].view(m, hidden)
    bg, bu, bd = banks
    lib.ffn_swiglu_q4k(dev(bg), dev(bu), dev(bd), dev(x), lib.Q4K_F32, m, hidden, inter, y,
                       workspace(lib, m, hidden, inter, k, 0), n_experts=n_exp, ids=dev(ids),
                       wts=dev(wts), top_k=k)
    ref = orc.moe_prefill(*banks, n_exp, hidden, inter, x, ids, wts)
    assert orc.relative_l2(host(y), ref) <= TOL
