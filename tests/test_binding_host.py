"""The Python binding rejects tensors of the wrong dtype or too few bytes before
anything reaches the library (runs without a GPU: the checks come before the
device check, and a CPU tensor that passes them is refused as not on the GPU)."""
import os

import pytest
import torch

import gemm_block_q4_amd as q4k
from gemm_block_q4_amd import _binding as B


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(B.library_path()):
        pytest.fail("libq4k.so is not built (run __graft_entry__.build())")
    return B.load_library()


def u8(n):
    return torch.empty(n, dtype=torch.uint8)


def f32(n):
    return torch.empty(n, dtype=torch.float32)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_gemv_sizes_and_dtypes():
    n, k, m = 16, 512, 2
    wb = q4k.q4k_weight_bytes(n, k)
    raises("w: holds", q4k.q4k_gemv, u8(wb - 1), f32(m * k), f32(m * n), m, n, k)
    raises("x: holds", q4k.q4k_gemv, u8(wb), f32(m * k - 1), f32(m * n), m, n, k)
    raises("y: holds", q4k.q4k_gemv, u8(wb), f32(m * k), f32(m * n - 1), m, n, k)
    raises("x: dtype", q4k.q4k_gemv, u8(wb), torch.empty(m * k, dtype=torch.float64), f32(m * n), m, n, k)
    raises("w: dtype", q4k.q4k_gemv, f32(wb), f32(m * k), f32(m * n), m, n, k)
    raises("must live on the GPU", q4k.q4k_gemv, u8(wb), f32(m * k), f32(m * n), m, n, k)
    raises("contiguous", q4k.q4k_gemv, u8(wb), f32(2 * m * k)[::2], f32(m * n), m, n, k)


def test_q8_1_and_mmq_sizes():
    m, n, k = 3, 8, 256
    raises("x: holds", q4k.q8_1_quantize, torch.empty(m * k - 1, dtype=torch.int16), q4k.Q4K_BF16, m, k,
           torch.empty(m * k, dtype=torch.int8), torch.empty(m * k // 32, dtype=torch.int32))
    raises("x: dtype", q4k.q8_1_quantize, f32(m * k), q4k.Q4K_BF16, m, k,
           torch.empty(m * k, dtype=torch.int8), torch.empty(m * k // 32, dtype=torch.int32))
    raises("ds: holds", q4k.q8_1_quantize, f32(m * k), q4k.Q4K_F32, m, k,
           torch.empty(m * k, dtype=torch.int8), torch.empty(m * k // 32 - 1, dtype=torch.int32))
    wb = q4k.q4k_weight_bytes(n, k)
    qs = torch.empty(m * k, dtype=torch.int8)
    ds = torch.empty(m * k // 32, dtype=torch.int32)
    raises("qs: holds", q4k.q4k_mmq, u8(wb), qs[:-1], ds, f32(m * n), m, n, k)
    raises("y: holds", q4k.q4k_mmq, u8(wb), qs, ds, f32(m * n - 1), m, n, k)
    raises("y: holds", q4k.q4k_mmq_bf16, u8(wb), qs, ds, torch.empty(m * n - 1, dtype=torch.int16), m, n, k)
    raises("y: dtype", q4k.q4k_mmq_bf16, u8(wb), qs, ds, f32(m * n), m, n, k)
    raises("ds: dtype", q4k.q4k_q8_gemv, u8(wb), qs, f32(m * k // 32), f32(m * n), m, n, k)
    raises("partials: holds", q4k.q4k_test_mmq_partials, u8(wb), qs, m, n, k,
           torch.empty(m * n * k // 32 - 1, dtype=torch.int32))


def test_quantize_and_q6k_sizes():
    rows, cols = 4, 512
    raises("w: holds", q4k.q4k_quantize, f32(rows * cols), q4k.Q4K_F32, rows, cols,
           u8(q4k.q4k_weight_bytes(rows, cols) - 1))
    raises("x: holds", q4k.q4k_quantize, torch.empty(rows * cols - 1, dtype=torch.int16), q4k.Q4K_BF16,
           rows, cols, u8(q4k.q4k_weight_bytes(rows, cols)))
    n, k = 5, 256
    raises("w: holds", q4k.q6k_gemv, u8(q4k.q6k_weight_bytes(n, k) - 1), f32(k), f32(n), n, k)
    raises("y: holds", q4k.q6k_gemv, u8(q4k.q6k_weight_bytes(n, k)), f32(k), f32(n - 1), n, k)


def test_ffn_sizes():
    m, hidden, inter = 2, 256, 512
    gu, dn = q4k.q4k_weight_bytes(inter, hidden), q4k.q4k_weight_bytes(hidden, inter)
    ws = u8(1024)
    args = dict(y=f32(m * hidden), workspace=ws)
    raises("w_up: holds", q4k.ffn_swiglu_q4k, u8(gu), u8(gu - 1), u8(dn), f32(m * hidden), q4k.Q4K_F32,
           m, hidden, inter, **args)
    raises("w_down: holds", q4k.ffn_swiglu_q4k, u8(gu), u8(gu), u8(dn - 1), f32(m * hidden), q4k.Q4K_F32,
           m, hidden, inter, **args)
    raises("x: holds", q4k.ffn_swiglu_q4k, u8(gu), u8(gu), u8(dn), f32(m * hidden - 1), q4k.Q4K_F32,
           m, hidden, inter, **args)
    # MoE: banks of n_experts matrices, ids / wts of m * top_k entries
    e, top_k = 3, 2
    ids = torch.empty(m * top_k, dtype=torch.int32)
    wts = f32(m * top_k)
    raises("w_gate: holds", q4k.ffn_swiglu_q4k, u8(e * gu - 1), u8(e * gu), u8(e * dn), f32(m * hidden),
           q4k.Q4K_F32, m, hidden, inter, n_experts=e, ids=ids, wts=wts, top_k=top_k, **args)
    raises("ids: holds", q4k.ffn_swiglu_q4k, u8(e * gu), u8(e * gu), u8(e * dn), f32(m * hidden),
           q4k.Q4K_F32, m, hidden, inter, n_experts=e, ids=ids[:-1], wts=wts, top_k=top_k, **args)
    raises("wts: dtype", q4k.ffn_swiglu_q4k, u8(e * gu), u8(e * gu), u8(e * dn), f32(m * hidden),
           q4k.Q4K_F32, m, hidden, inter, n_experts=e, ids=ids, wts=ids, top_k=top_k, **args)
    raises("must live on the GPU", q4k.ffn_swiglu_q4k, u8(e * gu), u8(e * gu), u8(e * dn),
           f32(m * hidden), q4k.Q4K_F32, m, hidden, inter, n_experts=e, ids=ids, wts=wts,
           top_k=top_k, **args)


def test_fp8_sizes():
    rows, cols = 3, 64
    raises("x: holds", q4k.fp8_absmax_rows, f32(rows * cols - 1), rows, cols, f32(rows))
    raises("absmax: holds", q4k.fp8_absmax_rows, f32(rows * cols), rows, cols, f32(rows - 1))
    raises("q: holds", q4k.fp8_quantize_rows, f32(rows * cols), rows, cols, f32(rows), u8(rows * cols - 1))
    raises("q: dtype", q4k.fp8_quantize_rows, f32(rows * cols), rows, cols, f32(rows), f32(rows * cols))
    m, n, k = 4, 8, 128
    raises("a: holds", q4k.fp8_gemm_dequant, u8(m * k - 1), f32(m), u8(n * k), f32(n), f32(m * n), m, n, k)
    raises("w_absmax: holds", q4k.fp8_gemm_dequant, u8(m * k), f32(m), u8(n * k), f32(n - 1), f32(m * n),
           m, n, k)
    raises("y: holds", q4k.fp8_gemm_dequant, u8(m * k), f32(m), u8(n * k), f32(n), f32(m * n - 1), m, n, k)
    raises("must live on the GPU", q4k.fp8_gemm_dequant, u8(m * k), f32(m), u8(n * k), f32(n), f32(m * n),
           m, n, k)


def test_library_loaded_first_shares_torch_hip_runtime():
    """Loading the library before anything imports torch still leaves one HIP
    runtime in the process (the library binds to torch's), so torch's streams
    and allocations are the library's too."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = ("import sys; sys.path.insert(0, %r)\n"
              "from gemm_block_q4_amd import _binding\n"
              "_binding.load_library()\n"
              "import torch\n"
              "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
              "print(len(maps))\n" % root)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    out = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout
