"""The allocation-free FFN entry point (ffn_swiglu_q4k_noalloc) against the
workspace entry point (ffn_swiglu_q4k) on the same inputs: both run the same
kernels, so the results must be equal bit for bit; the first call of each pair
is also checked against the oracle (relative L2 <= 2e-3).  Each case makes two
calls in a row, the second with a smaller input, so the second runs on the
scratch contents the first left behind."""
import numpy as np
import pytest
import torch

import gemm_block_q4_amd as q4kmod
from gemm_block_q4_amd import synth
from oracle import q4k_oracle as orc
from gpu_helpers import dev, empty, host, say, workspace

pytestmark = pytest.mark.gpu
TOL = 2e-3


def both(q4k, wg, wu, wd, x, hidden, inter, regime=0, bf16=False, n_exp=1, ids=None, wts=None):
    m = x.shape[0]
    top_k = 0 if ids is None else ids.shape[1]
    xin = dev(synth.to_bf16_bits(x).view(np.int16)) if bf16 else dev(x)
    xdt = q4k.Q4K_BF16 if bf16 else q4k.Q4K_F32
    dg, du, dd = dev(wg), dev(wu), dev(wd)
    di = None if ids is None else dev(ids)
    dw = None if wts is None else dev(wts)
    y_ws = empty((m, hidden), torch.float32)
    y_na = empty((m, hidden), torch.float32)
    ws = workspace(q4k, m, hidden, inter, top_k, regime)
    q4k.ffn_swiglu_q4k(dg, du, dd, xin, xdt, m, hidden, inter, y_ws, ws, n_experts=n_exp, ids=di,
                       wts=dw, top_k=top_k, regime=regime)
    q4k.ffn_swiglu_q4k_noalloc(dg, du, dd, xin, xdt, m, hidden, inter, y_na, n_experts=n_exp, ids=di,
                               wts=dw, top_k=top_k, regime=regime)
    return host(y_ws), host(y_na)


@pytest.mark.parametrize("regime", [q4kmod.Q4K_REGIME_DECODE, q4kmod.Q4K_REGIME_DECODE_Q8])
def test_noalloc_decode_two_calls(lib, regime):
    hidden, inter = 4096, 11008
    wg, wu, wd = synth.dense_ffn_weights(synth.DECODE_FFN_7B, hidden, inter)
    for call, m in enumerate((8, 1)):
        say(f"noalloc decode regime={regime} 4096/11008 m={m} (call {call + 1})")
        x = synth.activations(synth.DECODE_FFN_7B, m, hidden, outliers=True, sub=m)
        y_ws, y_na = both(lib, wg, wu, wd, x, hidden, inter, regime=regime)
        assert np.array_equal(y_ws, y_na)
        if call == 0:
            ref = (orc.ffn_decode if regime == q4kmod.Q4K_REGIME_DECODE else orc.ffn_prefill)(
                wg, wu, wd, hidden, inter, x)
            assert orc.relative_l2(y_na, ref) <= TOL


def test_noalloc_prefill_two_calls(lib):
    # 130 tokens at 512/1536 split the down pass over k (partial planes in
    # the scratch), then 9 tokens on what they left
    hidden, inter = 512, 1536
    wg, wu, wd = synth.dense_ffn_weights(91, hidden, inter)
    for call, m in enumerate((130, 9)):
        say(f"noalloc prefill 512/1536 m={m} (call {call + 1})")
        x = synth.activations(91, m, hidden, outliers=True, sub=m)
        y_ws, y_na = both(lib, wg, wu, wd, x, hidden, inter, regime=q4kmod.Q4K_REGIME_PREFILL, bf16=True)
        assert np.array_equal(y_ws, y_na)
        xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
        assert orc.relative_l2(y_na, orc.ffn_prefill(wg, wu, wd, hidden, inter, xb)) <= TOL


def test_noalloc_prefill_full_width(lib):
    # 512 tokens of the 5120/17408 prefill fit the scratch (48.6 MB), then 64
    say("noalloc prefill 5120/17408 m=512, then m=64")
    hidden, inter = 5120, 17408
    wg, wu, wd = synth.dense_ffn_weights(synth.PREFILL_FFN, hidden, inter)
    for m in (512, 64):
        x = synth.activations(synth.PREFILL_FFN, m, hidden, outliers=True, sub=m)
        y_ws, y_na = both(lib, wg, wu, wd, x, hidden, inter, bf16=True)
        assert np.array_equal(y_ws, y_na)


def test_noalloc_moe_two_calls(lib):
    n_exp, hidden, inter, k = 64, 2048, 768, 8
    banks = synth.moe_banks(synth.MOE_DECODE, n_exp, hidden, inter)
    for call, m in enumerate((4, 2)):
        say(f"noalloc moe 64 x top-8 2048/768 m={m} (call {call + 1})")
        x = synth.activations(synth.MOE_DECODE, m, hidden, outliers=False, sub=m)
        ids, wts = synth.router(synth.MOE_DECODE, m, n_exp, k, seed=call)
        y_ws, y_na = both(lib, *banks, x, hidden, inter, n_exp=n_exp, ids=ids, wts=wts)
        assert np.array_equal(y_ws, y_na)
        assert orc.relative_l2(y_na, orc.moe_decode(*banks, n_exp, hidden, inter, x, ids, wts)) <= TOL


def test_noalloc_moe_prefill_two_calls(lib):
    # MoE above 8 tokens: the grouped prefill passes, their pair list, tile
    # table and tile count in the scratch; the second call routes other pairs
    n_exp, hidden, inter, k = 64, 2048, 768, 8
    banks = synth.moe_banks(synth.MOE_DECODE, n_exp, hidden, inter)
    for call, m in enumerate((200, 33)):
        say(f"noalloc moe prefill 64 x top-8 2048/768 m={m} (call {call + 1})")
        x = synth.activations(synth.MOE_DECODE, m, hidden, outliers=True, sub=m + 1)
        ids, wts = synth.router(synth.MOE_DECODE, m, n_exp, k, seed=m)
        y_ws, y_na = both(lib, *banks, x, hidden, inter, n_exp=n_exp, ids=ids, wts=wts)
        assert np.array_equal(y_ws, y_na)
        toks = [0, m // 2, m - 1]
        ref = orc.moe_prefill(*banks, n_exp, hidden, inter, x, ids, wts, tokens=toks)
        assert orc.relative_l2(y_na[toks], ref) <= TOL


def test_noalloc_refuses_oversized_layout(lib):
    # 4096 prefill tokens of 5120/17408 need more than the fixed scratch:
    # refused before any launch
    say("noalloc refuses an oversized layout")
    m, hidden, inter = 4096, 5120, 17408
    assert lib.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter) > lib.Q4K_NOALLOC_SCRATCH_BYTES
    w = empty((lib.q4k_weight_bytes(inter, hidden),), torch.uint8)
    wd = empty((lib.q4k_weight_bytes(hidden, inter),), torch.uint8)
    x = empty((m, hidden), torch.int16)
    y = empty((m, hidden), torch.float32)
    with pytest.raises(lib.Q4KError) as e:
        lib.ffn_swiglu_q4k_noalloc(w, w, wd, x, lib.Q4K_BF16, m, hidden, inter, y)
    assert e.value.status == 8
