"""Seeded synthetic inputs for the Q4_K FFN workloads (numpy only).

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no dequantisation, no quantisation, no dot products), so
both the HIP path and the CPU oracle can be fed from it.

Every stream is ``numpy.random.Generator(PCG64(SeedSequence([seed, workload,
tensor, sub])))``.  Tensor ids: 0 activations, 1 gate, 2 up, 3 down,
4 router ids, 5 router logits, 6 outlier positions.

Q4_K blocks follow the workload description: every 4-bit quant uniform on
0..15, every 6-bit scale and min uniform on 0..63, and ``d``, ``dmin`` the
binary16 rounding of a uniform draw on [1e-3, 1e-2].  The twelve scale bytes
pack sixteen 6-bit fields one-to-one, so sixteen independent uniform 6-bit
values are exactly twelve independent uniform bytes, and 256 uniform nibbles
are 128 uniform bytes; the generator draws those bytes directly.
"""

from __future__ import annotations

import numpy as np

BLOCK_WEIGHTS = 256
BLOCK_BYTES = 144

TENSOR_X, TENSOR_GATE, TENSOR_UP, TENSOR_DOWN = 0, 1, 2, 3
TENSOR_ROUTER_IDS, TENSOR_ROUTER_LOGITS, TENSOR_OUTLIERS = 4, 5, 6


def rng(workload: int, tensor: int, sub: int = 0, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload, tensor, sub])))


def random_q4k(g: np.random.Generator, rows: int, cols: int,
               dlo: float = 1e-3, dhi: float = 1e-2) -> np.ndarray:
    """Random block_q4_K matrix [rows, cols] as uint8 [rows * cols/256 * 144]."""
    if cols % BLOCK_WEIGHTS:
        raise ValueError("cols must be a multiple of 256")
    nb = rows * (cols // BLOCK_WEIGHTS)
    d = g.uniform(dlo, dhi, nb).astype(np.float32).astype(np.float16)
    dmin = g.uniform(dlo, dhi, nb).astype(np.float32).astype(np.float16)
    scales = g.integers(0, 256, (nb, 12), dtype=np.uint8)
    quants = g.integers(0, 256, (nb, 128), dtype=np.uint8)
    out = np.empty((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = scales
    out[:, 16:144] = quants
    return out.reshape(-1)


Q6K_BLOCK_BYTES = 210


def random_q6k(g: np.random.Generator, rows: int, cols: int,
               dlo: float = 1e-3, dhi: float = 1e-2) -> np.ndarray:
    """Random block_q6_K matrix [rows, cols] as uint8 [rows * cols/256 * 210]:
    208 uniform bytes (the 4-bit and 2-bit quant fields, then 16 int8 scales)
    and a binary16 d drawn uniform on [dlo, dhi]."""
    if cols % BLOCK_WEIGHTS:
        raise ValueError("cols must be a multiple of 256")
    nb = rows * (cols // BLOCK_WEIGHTS)
    body = g.integers(0, 256, (nb, 208), dtype=np.uint8)
    d = g.uniform(dlo, dhi, nb).astype(np.float32).astype(np.float16)
    out = np.empty((nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :208] = body
    out[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def activations(workload: int, m: int, k: int, outliers: bool, sub: int = 0,
                seed: int = 0) -> np.ndarray:
    """f32 [m, k] from N(0, 1); with ``outliers`` exactly max(1, round(0.001*m*k))
    distinct entries are multiplied by 100."""
    x = rng(workload, TENSOR_X, sub, seed).standard_normal((m, k)).astype(np.float32)
    if outliers and m * k > 0:
        count = max(1, int(round(0.001 * m * k)))
        pos = rng(workload, TENSOR_OUTLIERS, sub, seed).choice(m * k, count, replace=False)
        flat = x.reshape(-1)
        flat[pos] = flat[pos] * np.float32(100.0)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 to bfloat16 (nearest, ties to even); returns the uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router(workload: int, m: int, n_experts: int, top_k: int, seed: int = 0):
    """Per token: top_k distinct expert ids (sorted) and softmax routing weights.

    Returns ids int32 [m, top_k] and weights f32 [m, top_k] (softmax of N(0,1)
    logits, computed in f64 then rounded).
    """
    g = rng(workload, TENSOR_ROUTER_IDS, 0, seed)
    ids = np.stack([np.sort(g.choice(n_experts, top_k, replace=False)) for _ in range(m)]).astype(np.int32)
    logits = rng(workload, TENSOR_ROUTER_LOGITS, 0, seed).standard_normal((m, top_k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.reshape(m, top_k), w


# -- the five workloads --------------------------------------------------------

TINY_FFN = 0          # hidden 256, inter 768, 1 token
GEMV_SWEEP = 1        # (n, k) in {(4096, 4096), (11008, 4096), (4096, 11008)}, 1 token
DECODE_FFN_7B = 2     # hidden 4096, inter 11008, 1/4/8 tokens, outliers
PREFILL_FFN = 3       # hidden 5120, inter 17408, 512/2048 tokens, bf16, outliers
MOE_DECODE = 4        # 64 experts, top-8, 4 tokens, hidden 2048, inter 768
LM_HEAD = 5           # Q6_K LM head GEMV: vocab 32000 x hidden 4096, 1 token
FP8_PREFILL = 6       # per-row FP8 recipe on the prefill FFN shapes (f32 weights)

GEMV_SWEEP_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))


def dense_ffn_weights(workload: int, hidden: int, inter: int, seed: int = 0):
    """Gate and up [inter, hidden], down [hidden, inter] as Q4_K bytes."""
    wg = random_q4k(rng(workload, TENSOR_GATE, 0, seed), inter, hidden)
    wu = random_q4k(rng(workload, TENSOR_UP, 0, seed), inter, hidden)
    wd = random_q4k(rng(workload, TENSOR_DOWN, 0, seed), hidden, inter)
    return wg, wu, wd


def moe_banks(workload: int, n_experts: int, hidden: int, inter: int, seed: int = 0):
    """Expert banks: expert e's matrix is the e-th consecutive matrix of its bank."""
    bg = random_q4k(rng(workload, TENSOR_GATE, 0, seed), n_experts * inter, hidden)
    bu = random_q4k(rng(workload, TENSOR_UP, 0, seed), n_experts * inter, hidden)
    bd = random_q4k(rng(workload, TENSOR_DOWN, 0, seed), n_experts * hidden, inter)
    return bg, bu, bd


def gemv_sweep_case(shape_index: int, m: int = 1, seed: int = 0):
    n, k = GEMV_SWEEP_SHAPES[shape_index]
    w = random_q4k(rng(GEMV_SWEEP, TENSOR_GATE, shape_index, seed), n, k)
    x = activations(GEMV_SWEEP, m, k, outliers=False, sub=shape_index, seed=seed)
    return n, k, w, x


def lm_head_case(vocab: int = 32000, hidden: int = 4096, sub: int = 0, seed: int = 0):
    """Q6_K LM head [vocab, hidden] and one N(0, 1) token."""
    w = random_q6k(rng(LM_HEAD, TENSOR_GATE, sub, seed), vocab, hidden)
    x = activations(LM_HEAD, 1, hidden, outliers=False, sub=sub, seed=seed)
    return w, x


def fp8_case(m: int, n: int, k: int, sub: int = 0, seed: int = 0):
    """Per-row FP8 GEMM inputs: activations f32 [m, k] N(0, 1) with 0.1%
    outliers x100 (as the prefill FFN's) and an f32 weight [n, k] N(0, 0.02)."""
    x = activations(FP8_PREFILL, m, k, outliers=True, sub=sub, seed=seed)
    w = (rng(FP8_PREFILL, TENSOR_GATE, sub, seed).standard_normal((n, k)) * 0.02).astype(np.float32)
    return x, w
