"""Throughput of the Q4_K FFN hot path on one MI355X.

Headline (``value``): effective weight-GB/s of the decode GEMV sweep, batch 1,
Q4_K weights [n, k] with (n, k) in {(4096, 4096), (11008, 4096),
(4096, 11008)}.  One step is one pass over the three GEMVs.  Weight bytes are
the algorithmic 144 bytes per 256 weights.  Every step reads a different copy
of each matrix (copies totalling >= 1 GiB per shape, four times the 256 MB
Infinity Cache), inputs are resident in HBM before timing starts, and the K
timed steps (and the W warmup steps) are each replayed from one HIP graph so
that host launch overhead is not measured.

Also reported (``secondary``): the 7B-style decode FFN at 1/4/8 tokens, the
prefill FFN (Q8_1 + MMQ) at 512 and 2048 tokens in TOPS, the 64-expert top-8
MoE decode FFN, the Q8_1-activation GEMV (q4k_q8_gemv) on the sweep shapes at
1/4/8 tokens, the load-time Q4_K quantiser, and the roofline of the dominant
kernel with the plain-read ceiling of the same bytes (q4k_test_read) beside
it.  Every per-call figure is the median of 5 replays of a graph of calls.
``cpu_baseline`` times the CPU oracle on a bounded sample of the headline
workload, on all BLAS threads and on one, with the host's CPU model and core
count.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5033.0        # dense int8 MFMA: 256 CU x 2.4 GHz x 8192 ops/clk
FP8_PEAK_TFLOPS = 5033.0       # dense FP8 MFMA: the same 8192 flop/clk per compute unit
ROTATE_BYTES = 1 << 30         # per rotated tensor set

# HBM bytes of one sweep (the three GEMV launches), measured with rocprofv3 FETCH_SIZE and
# WRITE_SIZE (each scaled by what it reads for a copy of known size; summary and commands in
# profiles/gemv_d4_decode_sweep_hbm_traffic.md) for the kernel sources with these SHA-256
# digests.  Reported only while the sources still match.
TRAFFIC_SWEEP_BYTES = 61117852
TRAFFIC_SOURCES = {
    "gemm_block_q4_amd/csrc/gemv_valu.hip":
        "17a03dc5cb645b393d6de1bc386efa643139a3b66631c8900087756d6e6eb327",
    "gemm_block_q4_amd/csrc/slice_dot.hpp":
        "2537bd57a417fc0675d828787fd917af1b119de52e1be70ef9f0d7168421d428",
    "gemm_block_q4_amd/csrc/lane_reduce.hpp":
        "81cf704adbded368721e276da797c733493ebe02c36c41b124b78709d1f364e1",
    "gemm_block_q4_amd/csrc/q4k_device.hpp":
        "532c6e881bd56ddab7a0e075b479fbab8468380451639a48865dc41a8cb9352e",
}


# the kernel the roofline describes (one token, dense): layout 1 (a row is one
# wavefront) for k = 4096, layout 2 (a row spans wavefronts) for k = 11008
GEMV_KERNEL = ("gemv_d4_kernel<false, false, 0, 1, 1, 4> for k = 4096 and "
               "gemv_d4_kernel<false, false, 0, 2, 1, 2> for k = 11008 (q4k_gemv, m = 1)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (where the library launches)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def capture(fn, count):
    """A HIP graph holding `count` calls fn(i)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)                      # eager run before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    torch.cuda.synchronize()
    return g


def rotated(tensor_np, total=ROTATE_BYTES, max_copies=None):
    """Device copies of one byte array so that copies * size >= total."""
    import torch
    nbytes = tensor_np.nbytes
    copies = max(2, -(-total // nbytes))
    if max_copies:
        copies = min(copies, max_copies)
    base = torch.from_numpy(np.ascontiguousarray(tensor_np)).cuda()
    stride = -(-nbytes // 256) * 256
    buf = torch.empty(copies * stride, dtype=torch.uint8, device="cuda")
    views = []
    for c in range(copies):
        v = buf[c * stride: c * stride + nbytes]
        v.copy_(base)
        views.append(v)
    return views


def measured_traffic():
    """TRAFFIC_SWEEP_BYTES if the GEMV sources are the measured ones, else None."""
    import hashlib
    for rel, digest in TRAFFIC_SOURCES.items():
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                data = f.read()
        except OSError:
            return None
        if hashlib.sha256(data).hexdigest() != digest:
            return None
    return TRAFFIC_SWEEP_BYTES


def timed_graph(fn, steps, warmup):
    g_w = capture(fn, max(1, warmup)) if warmup > 0 else None
    g_t = capture(fn, steps)
    if g_w is not None:
        g_w.replay()
    with Timer() as t:
        g_t.replay()
    return t.ms


TRIALS = 5


def median_us(fn, reps, trials=TRIALS):
    """Median over `trials` replays of one graph of `reps` calls fn(i) (after
    one untimed replay): microseconds per call, with the trials' spread."""
    g = capture(fn, reps)
    g.replay()
    per = []
    for _ in range(trials):
        with Timer() as t:
            g.replay()
        per.append(t.ms * 1e3 / reps)
    per.sort()
    return per[len(per) // 2], per[0], per[-1]


# -- headline: GEMV sweep -----------------------------------------------------------

def gemv_sweep(q4k, synth, steps, warmup):
    import torch
    shapes = []
    for s, (n, k) in enumerate(synth.GEMV_SWEEP_SHAPES):
        _, _, w, x = synth.gemv_sweep_case(s)
        shapes.append(dict(n=n, k=k, w=rotated(w), x=torch.from_numpy(x).cuda(),
                           y=torch.empty((1, n), dtype=torch.float32, device="cuda"),
                           bytes=q4k.q4k_weight_bytes(n, k)))

    def one_pass(i):
        for sh in shapes:
            ws = sh["w"][i % len(sh["w"])]
            q4k.q4k_gemv(ws, sh["x"], sh["y"], 1, sh["n"], sh["k"])

    ms = timed_graph(one_pass, steps, warmup)
    total_bytes = steps * sum(sh["bytes"] for sh in shapes)
    # per-shape launch duration (median of 5 replays of a graph of launches
    # of one shape over the rotated copies), and the plain-read ceiling: the
    # same bytes of the same copies streamed by q4k_test_read
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    per_shape = []
    for sh in shapes:
        reps = len(sh["w"])

        def one(i, sh=sh):
            q4k.q4k_gemv(sh["w"][i % len(sh["w"])], sh["x"], sh["y"], 1, sh["n"], sh["k"])

        def read(i, sh=sh):
            q4k.q4k_test_read(sh["w"][i % len(sh["w"])], sh["bytes"], sink)

        us, us_lo, us_hi = median_us(one, reps)
        rd, _, _ = median_us(read, reps)
        per_shape.append(dict(n=sh["n"], k=sh["k"], bytes=sh["bytes"], us=us, us_min=us_lo, us_max=us_hi,
                              gbs=sh["bytes"] / (us * 1e-6) / 1e9, read_us=rd,
                              read_gbs=sh["bytes"] / (rd * 1e-6) / 1e9))
    return ms, total_bytes, per_shape


# -- secondary workloads -------------------------------------------------------------

def decode_ffn(q4k, synth, reps=40):
    import torch
    hidden, inter = 4096, 11008
    wg, wu, wd = synth.dense_ffn_weights(synth.DECODE_FFN_7B, hidden, inter)
    per_ffn = 2 * q4k.q4k_weight_bytes(inter, hidden) + q4k.q4k_weight_bytes(hidden, inter)
    cat = np.concatenate([wg, wu, wd])
    copies = rotated(cat)
    gb = q4k.q4k_weight_bytes(inter, hidden)
    out = {}
    # f32 activations (the decode regime), then the Q8_1 decode regime
    # (Q8_1 of x and h, integer-dot GEMVs; entries "q8_m1" ...)
    for tag, regime in (("", q4k.Q4K_REGIME_DECODE), ("q8_", q4k.Q4K_REGIME_DECODE_Q8)):
        for m in (1, 4, 8):
            x = torch.from_numpy(synth.activations(synth.DECODE_FFN_7B, m, hidden, True, sub=m)).cuda()
            y = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
            ws = torch.empty(q4k.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter, 0, regime),
                             dtype=torch.uint8, device="cuda")

            def call(i, x=x, y=y, ws=ws, m=m, regime=regime):
                c = copies[i % len(copies)]
                q4k.ffn_swiglu_q4k(c[:gb], c[gb:2 * gb], c[2 * gb:], x, q4k.Q4K_F32, m, hidden, inter,
                                   y, ws, regime=regime)

            us, _, _ = median_us(call, reps)
            out[f"{tag}m{m}"] = dict(us_per_ffn=round(us, 2), tokens_per_s=round(m / (us * 1e-6), 1),
                                     weight_gbs=round(per_ffn / (us * 1e-6) / 1e9, 1))
    return out


def q8_gemv(q4k, synth):
    """Q8_1-activation decode GEMV (q4k_q8_gemv) on the sweep shapes at 1, 4 and
    8 tokens: average launch time over a graph of launches on rotated weight
    copies, and effective weight-GB/s.  The activations are quantised once by
    q8_1_quantize before timing."""
    import torch
    out = {}
    for s, (n, k) in enumerate(synth.GEMV_SWEEP_SHAPES):
        _, _, w, _ = synth.gemv_sweep_case(s)
        copies = rotated(w)
        nbytes = q4k.q4k_weight_bytes(n, k)
        for m in (1, 4, 8):
            x = torch.from_numpy(synth.activations(synth.GEMV_SWEEP, m, k, True, sub=100 + m)).cuda()
            qs = torch.empty((m, k), dtype=torch.int8, device="cuda")
            ds = torch.empty((m, k // 32), dtype=torch.int32, device="cuda")
            q4k.q8_1_quantize(x, q4k.Q4K_F32, m, k, qs, ds)
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")

            def call(i, copies=copies, qs=qs, ds=ds, y=y, m=m, n=n, k=k):
                q4k.q4k_q8_gemv(copies[i % len(copies)], qs, ds, y, m, n, k)

            us, _, _ = median_us(call, len(copies))
            out[f"n{n}_k{k}_m{m}"] = dict(us=round(us, 2), weight_gbs=round(nbytes / (us * 1e-6) / 1e9, 1))
    return out


def quantize_q4k(q4k, synth):
    """Load-time Q4_K quantiser (q4k_quantize) on the [11008, 4096] matrix from
    f32 and from bf16: average launch time over a graph of launches on rotated
    input copies (>= 1 GiB), and GB/s of input plus output bytes."""
    import torch
    rows, cols = 11008, 4096
    x = synth.activations(synth.GEMV_SWEEP, rows, cols, False, sub=200)
    out_bytes = q4k.q4k_weight_bytes(rows, cols)
    w = torch.empty(out_bytes, dtype=torch.uint8, device="cuda")
    res = {}
    for name, arr, dt in (("f32", x, q4k.Q4K_F32), ("bf16", synth.to_bf16_bits(x), q4k.Q4K_BF16)):
        raw = rotated(arr.view(np.uint8).reshape(-1))
        src = [c.view(torch.float32 if dt == q4k.Q4K_F32 else torch.int16) for c in raw]

        def call(i, src=src, dt=dt):
            q4k.q4k_quantize(src[i % len(src)], dt, rows, cols, w)

        us, _, _ = median_us(call, len(src))
        moved = arr.nbytes + out_bytes
        res[name] = dict(us=round(us, 2), gbs=round(moved / (us * 1e-6) / 1e9, 1))
    return res


def lm_head_q6k(q4k, synth):
    """Q6_K LM head GEMV (q6k_gemv), vocab 32000 x hidden 4096, one token:
    average launch time over a graph of launches on rotated weight copies
    (>= 1 GiB), and effective weight-GB/s (210 B per 256 weights)."""
    import torch
    n, k = 32000, 4096
    w, x = synth.lm_head_case(n, k)
    copies = rotated(w)
    xd = torch.from_numpy(x.reshape(-1)).cuda()
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    nbytes = q4k.q6k_weight_bytes(n, k)

    def call(i):
        q4k.q6k_gemv(copies[i % len(copies)], xd, y, n, k)

    us, _, _ = median_us(call, 4 * len(copies))
    return dict(us=round(us, 2), weight_gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac_hbm_peak=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))


def mmq_store(q4k, synth, reps=4):
    """Single-matrix MMQ (the prefill down projection's shape, [5120, 17408],
    2048 tokens, no k split) with the f32 store (q4k_mmq) and the fused
    bfloat16 store (q4k_mmq_bf16): average launch time over a graph of
    launches on rotated weight copies, and TOPS."""
    import torch
    n, k, m = 5120, 17408, 2048
    w = synth.random_q4k(synth.rng(synth.PREFILL_FFN, 3, 7), n, k)
    copies = rotated(w, max_copies=7)
    x = torch.from_numpy(synth.activations(synth.PREFILL_FFN, m, k, True, sub=7)).cuda()
    qs = torch.empty((m, k), dtype=torch.int8, device="cuda")
    ds = torch.empty((m, k // 32), dtype=torch.int32, device="cuda")
    q4k.q8_1_quantize(x, q4k.Q4K_F32, m, k, qs, ds)
    y32 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    y16 = torch.empty((m, n), dtype=torch.int16, device="cuda")
    out = {}
    for name, fn, y in (("f32", q4k.q4k_mmq, y32), ("bf16", q4k.q4k_mmq_bf16, y16)):
        def call(i, fn=fn, y=y):
            fn(copies[i % len(copies)], qs, ds, y, m, n, k)

        us, _, _ = median_us(call, reps)
        out[name] = dict(us=round(us, 1), tops=round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1))
    return out


def prefill_ffn(q4k, synth, reps=4):
    import torch
    hidden, inter = 5120, 17408
    wg, wu, wd = synth.dense_ffn_weights(synth.PREFILL_FFN, hidden, inter)
    gb = q4k.q4k_weight_bytes(inter, hidden)
    copies = rotated(np.concatenate([wg, wu, wd]), max_copies=7)
    out = {}
    for m in (512, 2048):
        xb = synth.to_bf16_bits(synth.activations(synth.PREFILL_FFN, m, hidden, True, sub=m))
        x = torch.from_numpy(xb.view(np.int16)).cuda()
        y = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
        ws = torch.empty(q4k.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter), dtype=torch.uint8,
                         device="cuda")

        def call(i):
            c = copies[i % len(copies)]
            q4k.ffn_swiglu_q4k(c[:gb], c[gb:2 * gb], c[2 * gb:], x, q4k.Q4K_BF16, m, hidden, inter,
                               y, ws)

        us, _, _ = median_us(call, reps)
        ops = 2.0 * m * (3 * hidden * inter)
        out[f"m{m}"] = dict(us_per_ffn=round(us, 1), tops=round(ops / (us * 1e-6) / 1e12, 1),
                            frac_int8_peak=round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                            tokens_per_s=round(m / (us * 1e-6), 1))
    return out


def moe_ffn(q4k, synth, reps=40):
    import torch
    n_exp, hidden, inter, m, k = 64, 2048, 768, 4, 8
    bg, bu, bd = synth.moe_banks(synth.MOE_DECODE, n_exp, hidden, inter)
    x = torch.from_numpy(synth.activations(synth.MOE_DECODE, m, hidden, False)).cuda()
    ids_np, wts_np = synth.router(synth.MOE_DECODE, m, n_exp, k)
    ids = torch.from_numpy(ids_np).cuda()
    wts = torch.from_numpy(wts_np).cuda()
    distinct = len(np.unique(ids_np))
    per_expert = 3 * q4k.q4k_weight_bytes(inter, hidden)
    bank = q4k.q4k_weight_bytes(inter, hidden) * n_exp
    copies = rotated(np.concatenate([bg, bu, bd]))
    y = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(q4k.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter, k), dtype=torch.uint8,
                     device="cuda")

    def call(i):
        c = copies[i % len(copies)]
        q4k.ffn_swiglu_q4k(c[:bank], c[bank:2 * bank], c[2 * bank:], x, q4k.Q4K_F32, m, hidden,
                           inter, y, ws, n_experts=n_exp, ids=ids, wts=wts, top_k=k)

    us, _, _ = median_us(call, reps)
    return dict(distinct_experts=distinct, us_per_ffn=round(us, 2),
                tokens_per_s=round(m / (us * 1e-6), 1),
                weight_gbs=round(distinct * per_expert / (us * 1e-6) / 1e9, 1))


def moe_prefill(q4k, synth, reps=6):
    """Top-k MoE FFN in the prefill regime (grouped MMQ passes): the routed
    workload's 64 experts, top-8, 2048/768, at 512 and 2048 tokens; TOPS over
    the pairs' 2 * 3 * hidden * inter ops each, on rotated bank copies."""
    import torch
    n_exp, hidden, inter, k = 64, 2048, 768, 8
    bg, bu, bd = synth.moe_banks(synth.MOE_DECODE, n_exp, hidden, inter)
    bank = q4k.q4k_weight_bytes(inter, hidden) * n_exp
    copies = rotated(np.concatenate([bg, bu, bd]), max_copies=6)
    out = {}
    for m in (512, 2048):
        x = torch.from_numpy(synth.activations(synth.MOE_DECODE, m, hidden, True, sub=m)).cuda()
        ids_np, wts_np = synth.router(synth.MOE_DECODE, m, n_exp, k, seed=m)
        ids = torch.from_numpy(ids_np).cuda()
        wts = torch.from_numpy(wts_np).cuda()
        y = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
        ws = torch.empty(q4k.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter, k), dtype=torch.uint8,
                         device="cuda")

        def call(i):
            c = copies[i % len(copies)]
            q4k.ffn_swiglu_q4k(c[:bank], c[bank:2 * bank], c[2 * bank:], x, q4k.Q4K_F32, m, hidden,
                               inter, y, ws, n_experts=n_exp, ids=ids, wts=wts, top_k=k)

        us, _, _ = median_us(call, reps)
        ops = 2.0 * m * k * 3 * hidden * inter
        out[f"m{m}"] = dict(us_per_ffn=round(us, 1), tops=round(ops / (us * 1e-6) / 1e12, 1),
                            frac_int8_peak=round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                            tokens_per_s=round(m / (us * 1e-6), 1))
    return out


def fp8_recipe(q4k, synth, reps=6):
    """Per-row FP8 recipe on the prefill FFN's projection shapes (gate/up
    [17408, 5120] and down [5120, 17408]) at 512 and 2048 tokens: the
    activation quantiser (row absmax + E4M3 codes, f32 x) and the FP8 GEMM
    with the outer dequant (f32 y), weights quantised once beforehand.
    Average launch times over graphs of launches on rotated weight copies;
    GEMM TFLOP/s against the dense FP8 matrix-core peak."""
    import torch
    out = {}
    for n, k, name in ((17408, 5120, "gate_up"), (5120, 17408, "down")):
        _, w = synth.fp8_case(1, n, k, sub=n)
        wd = torch.from_numpy(w).cuda()
        wam = torch.empty(n, dtype=torch.float32, device="cuda")
        qw = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        q4k.fp8_absmax_rows(wd, n, k, wam)
        q4k.fp8_quantize_rows(wd, n, k, wam, qw)
        del wd
        copies = [qw] + [qw.clone() for _ in range(3)]
        for m in (512, 2048):
            x = torch.from_numpy(synth.fp8_case(m, 1, k, sub=m)[0]).cuda()
            am = torch.empty(m, dtype=torch.float32, device="cuda")
            qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")

            def quant(i):
                q4k.fp8_absmax_rows(x, m, k, am)
                q4k.fp8_quantize_rows(x, m, k, am, qa)

            def gemm(i):
                q4k.fp8_gemm_dequant(qa, am, copies[i % len(copies)], wam, y, m, n, k)

            quant(0)
            q_us, _, _ = median_us(quant, 4 * reps)
            g_us, g_min, g_max = median_us(gemm, 4 * reps)
            tflops = 2.0 * m * n * k / (g_us * 1e-6) / 1e12
            out[f"{name}_m{m}"] = dict(quantize_us=round(q_us, 1), gemm_us=round(g_us, 1),
                                       gemm_us_min=round(g_min, 1), gemm_us_max=round(g_max, 1),
                                       gemm_tflops=round(tflops, 1),
                                       frac_fp8_peak=round(tflops / FP8_PEAK_TFLOPS, 4))
    return out


# -- CPU oracle baseline ---------------------------------------------------------------

def cpu_info():
    """Host CPU model (from /proc/cpuinfo, as lscpu reports it) and the cores this
    process may run on (what nproc prints)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_oracle_rate(orc, cases, seconds):
    """Weight-GB/s of the oracle GEMV over passes of the sweep for about `seconds`."""
    total = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        for n, k, w, x in cases:
            orc.gemv(w, n, k, x)
            total += orc.q4k_weight_bytes(n, k)
        passes += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return total / dt / 1e9, passes, dt


def cpu_baseline(synth):
    """The f64 numpy oracle (dequantise, then a BLAS matrix-vector product) on
    the batch-1 GEMV sweep, once with every BLAS thread of the host and once
    on one thread.  The oracle is a correctness reference, untuned."""
    from oracle import q4k_oracle as orc
    from threadpoolctl import threadpool_info, threadpool_limits
    model, nproc = cpu_info()
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cases = [synth.gemv_sweep_case(s) for s in range(3)]
    all_rate, all_passes, all_dt = cpu_oracle_rate(orc, cases, 8.0)
    with threadpool_limits(limits=1):
        one_rate, one_passes, one_dt = cpu_oracle_rate(orc, cases, 8.0)
    return dict(value=round(all_rate, 3), unit="GB/s", cores=blas_threads, kind="oracle",
                sample=f"{all_passes} pass(es) of the 3-shape batch-1 GEMV sweep through the f64 "
                       f"numpy oracle (dequantise + matmul) on {blas_threads} BLAS threads, "
                       f"{all_dt:.1f} s; the dequantisation itself runs on one thread",
                single_thread=dict(value=round(one_rate, 3), unit="GB/s", cores=1,
                                   sample=f"{one_passes} pass(es), {one_dt:.1f} s"),
                nproc=nproc, cpu_model=model,
                note="plain f64 correctness oracle, not a tuned CPU kernel")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--secondary", default="",
                    help="comma-separated secondary workload keys to run (default: all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_block_q4_amd as q4k
    from gemm_block_q4_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q4k.load_library()
    torch.cuda.set_device(0)

    log("bench: GEMV sweep")
    ms, total_bytes, per_shape = gemv_sweep(q4k, synth, args.steps, args.warmup)
    value = total_bytes / (ms * 1e-3) / 1e9
    log(f"bench: GEMV sweep {value:.1f} GB/s over {args.steps} steps ({ms:.3f} ms)")

    sum_bytes = sum(p["bytes"] for p in per_shape)
    sum_us = sum(p["us"] for p in per_shape)
    sum_read = sum(p["read_us"] for p in per_shape)
    achieved = sum_bytes / (sum_us * 1e-6) / 1e9
    read_gbs = sum_bytes / (sum_read * 1e-6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                    traffic_scope="HBM bytes of the three sweep launches (same scope as achieved)",
                    kernel=GEMV_KERNEL,
                    timing=f"per shape: median of {TRIALS} replays of a graph of launches over the "
                           "rotated copies (HIP events on the launch stream)",
                    read_ceiling_gbs=round(read_gbs, 1),
                    frac_of_read_ceiling=round(achieved / read_gbs, 4),
                    read_ceiling_note="q4k_test_read: one 16-byte load per thread over the same "
                                      "bytes of the same copies, timed the same way; a 70% of 8 TB/s "
                                      "target below the read ceiling's time is out of reach of any "
                                      "single launch",
                    per_shape=[dict(n=p["n"], k=p["k"], us=round(p["us"], 3),
                                    us_min=round(p["us_min"], 3), us_max=round(p["us_max"], 3),
                                    gbs=round(p["gbs"], 1), read_us=round(p["read_us"], 3),
                                    read_gbs=round(p["read_gbs"], 1),
                                    frac_of_read_ceiling=round(p["read_us"] / p["us"], 4),
                                    target_us_70pct_hbm=round(p["bytes"] / (0.7 * HBM_PEAK_GBS * 1e3), 3))
                               for p in per_shape])

    secondary = {}
    if not args.skip_secondary:
        workloads = (
            ("decode_ffn_4096_11008", "decode FFN", decode_ffn),
            ("prefill_ffn_5120_17408", "prefill FFN", prefill_ffn),
            ("moe_64x_top8_2048_768", "MoE", moe_ffn),
            ("q8_gemv_sweep", "Q8_1-activation GEMV", q8_gemv),
            ("q4k_quantize_11008_4096", "Q4_K quantiser", quantize_q4k),
            ("mmq_store_5120_17408_m2048", "MMQ f32 and bf16 stores", mmq_store),
            ("lm_head_q6k_32000_4096", "Q6_K LM head GEMV", lm_head_q6k),
            ("moe_prefill_64x_top8_2048_768", "MoE prefill (grouped MMQ)", moe_prefill),
            ("fp8_recipe_5120_17408", "per-row FP8 recipe", fp8_recipe),
        )
        only = [w for w in args.secondary.split(",") if w] if args.secondary else []
        for key, what, fn in workloads:
            if only and key not in only:
                continue
            log(f"bench: {what}")
            secondary[key] = fn(q4k, synth)

    cpu = None
    if not args.skip_cpu:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(synth)

    line = {
        "metric": "Q4_K GEMV weight-GB/s (% HBM peak); MMQ prefill TOPS (% int8 MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode GEMV sweep, batch 1, Q4_K [n,k] in "
                               "{(4096,4096),(11008,4096),(4096,11008)}, x f32 N(0,1), seed 0",
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
