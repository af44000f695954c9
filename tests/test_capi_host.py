"""The C ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from gemm_block_q4_amd import _binding as B
from oracle import q4k_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4k.h")

# Fake, aligned, never dereferenced device addresses: every call below fails
# validation before the library touches the HIP runtime.
P = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        pytest.fail("libq4k.so is not built (run __graft_entry__.build())")
    return B.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"q4k_gemv", "q8_1_quantize", "q4k_mmq", "ffn_swiglu_q4k", "q4k_weight_bytes",
            "q4k_status_string", "ffn_swiglu_q4k_workspace_bytes",
            "q4k_test_mmq_partials", "q4k_q8_gemv", "q4k_quantize", "q6k_gemv",
            "q6k_weight_bytes", "q4k_mmq_bf16", "ffn_swiglu_q4k_noalloc",
            "q4k_test_read"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_weight_bytes_matches_oracle(lib):
    for rows, cols in ((768, 256), (4096, 11008), (17408, 5120), (2048, 768)):
        assert lib.q4k_weight_bytes(rows, cols) == orc.q4k_weight_bytes(rows, cols)
    assert lib.q4k_weight_bytes(4, 300) == 0
    assert lib.q4k_weight_bytes(-1, 256) == 0


def test_status_strings(lib):
    for s in range(0, 9):
        assert lib.q4k_status_string(s)
    assert lib.q4k_status_string(99) == b"unknown status"


def test_gemv_validation(lib):
    assert lib.q4k_gemv(None, P, P, 1, 16, 256, None) == 1
    assert lib.q4k_gemv(P, P, P, 0, 16, 256, None) == 2
    assert lib.q4k_gemv(P, P, P, 9, 16, 256, None) == 2
    assert lib.q4k_gemv(P, P, P, 1, 16, 300, None) == 2      # k not a multiple of 256
    assert lib.q4k_gemv(P, P, P, 1, 0, 256, None) == 2
    assert lib.q4k_gemv(P + 4, P, P, 1, 16, 256, None) == 3  # misaligned weights
    assert lib.q4k_gemv(P, P, P, 1, 1 << 30, 32768, None) == 4    # block count overflows
    assert lib.q4k_gemv(P, P, P, 1, 16, 32768 + 256, None) == 2   # k above the decode limit


def test_q8_1_validation(lib):
    assert lib.q8_1_quantize(None, 0, 1, 32, P, P, None) == 1
    assert lib.q8_1_quantize(P, 2, 1, 32, P, P, None) == 2
    assert lib.q8_1_quantize(P, 0, 1, 48, P, P, None) == 2
    assert lib.q8_1_quantize(P + 4, 0, 1, 32, P, P, None) == 3


def test_mmq_validation(lib):
    assert lib.q4k_mmq(P, None, P, P, 1, 1, 256, None) == 1
    assert lib.q4k_mmq(P, P, P, P, 1, 1, 512 + 32, None) == 2
    assert lib.q4k_mmq(P, P + 1, P, P, 1, 1, 256, None) == 3
    assert lib.q4k_test_mmq_partials(P, P, 1, 1, 256, None, None) == 1
    assert lib.q4k_mmq(P, P, P, P, 1, 1, (1 << 20) + 256, None) == 2  # k above the prefill limit


def test_q8_gemv_validation(lib):
    assert lib.q4k_q8_gemv(P, P, None, P, 1, 1, 256, None) == 1
    assert lib.q4k_q8_gemv(P, P, P, P, 0, 1, 256, None) == 2
    assert lib.q4k_q8_gemv(P, P, P, P, 9, 1, 256, None) == 2          # more than 8 tokens
    assert lib.q4k_q8_gemv(P, P, P, P, 1, 1, 512 + 32, None) == 2     # k not a multiple of 256
    assert lib.q4k_q8_gemv(P, P, P, P, 1, 1, 32768 + 256, None) == 2  # k above the decode limit
    assert lib.q4k_q8_gemv(P, P + 4, P, P, 1, 1, 256, None) == 3      # misaligned quants
    assert lib.q4k_q8_gemv(P, P, P + 4, P, 1, 1, 256, None) == 3      # misaligned scale words


def test_quantize_validation(lib):
    assert lib.q4k_quantize(None, 0, 1, 256, P, None) == 1
    assert lib.q4k_quantize(P, 0, 1, 256, None, None) == 1
    assert lib.q4k_quantize(P, 7, 1, 256, P, None) == 2          # unknown dtype
    assert lib.q4k_quantize(P, 0, 0, 256, P, None) == 2
    assert lib.q4k_quantize(P, 0, 1, 300, P, None) == 2          # cols not a multiple of 256
    assert lib.q4k_quantize(P + 4, 0, 1, 256, P, None) == 3      # f32 input needs 16 bytes
    assert lib.q4k_quantize(P + 8, 1, 1, 256, P, None) == 3      # bf16 input needs 16 bytes too
    assert lib.q4k_quantize(P, 1, 1, 256, P + 4, None) == 3      # misaligned output
    assert lib.q4k_quantize(P, 0, 1 << 30, 32768, P, None) == 4  # block count overflows


def test_ffn_validation(lib):
    f = lib.ffn_swiglu_q4k
    ws = lib.ffn_swiglu_q4k_workspace_bytes(1, 256, 768, 0, 0)
    assert ws > 0
    # null weights
    assert f(None, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 0, P, P, ws, None) == 1
    # hidden not a multiple of 256
    assert f(P, P, P, 1, P, 0, 1, 300, 768, None, None, 0, 0, P, P, ws, None) == 2
    # dense call with several experts
    assert f(P, P, P, 2, P, 0, 1, 256, 768, None, None, 0, 0, P, P, ws, None) == 2
    # MoE without routing weights
    assert f(P, P, P, 4, P, 0, 1, 256, 768, P, None, 2, 0, P, P, ws, None) == 1
    # MoE top_k larger than the expert count
    assert f(P, P, P, 4, P, 0, 1, 256, 768, P, P, 5, 0, P, P, ws, None) == 2
    # MoE in the prefill regime (grouped MMQ): needs its own, larger workspace,
    # at most 4096 experts (the routing counters) and 32-bit token-row offsets
    pre_ws = lib.ffn_swiglu_q4k_workspace_bytes(16, 256, 768, 2, 2)
    assert pre_ws > ws
    assert f(P, P, P, 4, P, 0, 1, 256, 768, P, P, 2, 2, P, P, ws, None) == 5
    assert f(P, P, P, 4, P, 0, 16, 256, 768, P, P, 2, 0, P, P, ws, None) == 5   # auto: 16 tokens
    assert f(P, P, P, 4097, P, 0, 16, 256, 768, P, P, 2, 2, P, P, 1 << 40, None) == 2
    assert f(P, P, P, 4, P, 0, 1 << 20, 4096, 768, P, P, 2, 2, P, P, 1 << 50, None) == 4
    assert f(P, P, P, 4, P, 0, 1 << 16, 256, 16384, P, P, 4, 2, P, P, 1 << 50, None) == 4
    # decode regime forced with too many tokens
    assert f(P, P, P, 1, P, 0, 9, 256, 768, None, None, 0, 1, P, P, ws, None) == 2
    # Q8_1 decode regime: at most 8 tokens, dense only, k bound of the decode GEMVs
    assert f(P, P, P, 1, P, 0, 9, 256, 768, None, None, 0, 3, P, P, ws, None) == 2
    assert f(P, P, P, 4, P, 0, 1, 256, 768, P, P, 2, 3, P, P, ws, None) == 2
    assert f(P, P, P, 1, P, 0, 1, 256, 32768 + 256, None, None, 0, 3, P, P, 1 << 40, None) == 2
    # unknown regime
    assert f(P, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 4, P, P, ws, None) == 2
    # Q8_1 decode regime with the f32 decode regime's (smaller) workspace
    assert lib.ffn_swiglu_q4k_workspace_bytes(1, 256, 768, 0, 3) > ws
    assert f(P, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 3, P, P, ws, None) == 5
    # workspace too small / missing
    assert f(P, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 0, P, P, ws - 1, None) == 5
    assert f(P, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 0, P, None, ws, None) == 5


def test_workspace_sizes(lib):
    w = lib.ffn_swiglu_q4k_workspace_bytes
    assert w(1, 4096, 11008, 0, 0) >= 11008 * 4
    assert w(8, 4096, 11008, 0, 0) >= 8 * 11008 * 4
    pre = w(512, 5120, 17408, 0, 0)
    assert pre >= 512 * (5120 + 5120 // 32 * 4 + 17408 * 4 + 17408 + 17408 // 32 * 4)
    assert w(4, 2048, 768, 8, 0) >= 32 * (768 + 2048) * 4
    # MoE rows wider than a wavefront (no expert-major combine counters)
    assert w(2, 512, 4608, 2, 0) >= 4 * (4608 + 512) * 4
    assert w(2, 8192, 512, 2, 0) >= 4 * (512 + 8192) * 4
    assert w(0, 256, 256, 0, 0) == 0
    assert w(9, 256, 256, 0, 1) == 0      # decode regime caps m at 8
    # MoE prefill: Q8_1(x), the sorted pair list and tile table, Q8_1(h) and
    # the f32 output of every pair
    assert w(4, 256, 256, 2, 2) >= 4 * (256 + 32) + 8 * (4 + 256 + 32 + 256 * 4)
    assert w(64, 2048, 768, 8, 0) >= 64 * (2048 + 256) + 512 * (4 + 768 + 96 + 2048 * 4)
    # Q8_1 decode: Q8_1 of x and of h, and h in f32
    assert w(8, 4096, 11008, 0, 3) >= 8 * (4096 + 4096 // 32 * 4 + 11008 * 4 + 11008 + 11008 // 32 * 4)
    assert w(9, 256, 256, 0, 3) == 0
    assert w(4, 256, 256, 2, 3) == 0      # MoE runs in the f32 decode regime only
    assert w(1, 256, 256, 0, 4) == 0


def test_q6k_sizes_and_validation(lib):
    from oracle import q6k_oracle as q6
    for rows, cols in ((32000, 4096), (1, 256), (7, 11008)):
        assert lib.q6k_weight_bytes(rows, cols) == q6.q6k_weight_bytes(rows, cols)
    assert lib.q6k_weight_bytes(4, 300) == 0
    assert lib.q6k_weight_bytes(-1, 256) == 0
    g = lib.q6k_gemv
    assert g(None, P, P, 10, 256, None) == 1
    assert g(P, None, P, 10, 256, None) == 1
    assert g(P, P, P, 0, 256, None) == 2           # no rows
    assert g(P, P, P, 10, 300, None) == 2          # k not a multiple of 256
    assert g(P, P, P, 10, 32768 + 256, None) == 2  # k above the decode bound
    assert g(P + 2, P, P, 10, 256, None) == 3      # weights need 16 bytes
    assert g(P, P + 4, P, 10, 256, None) == 3      # x needs 16 bytes
    assert g(P, P, P + 2, 10, 256, None) == 3
    assert g(P, P, P, 1 << 30, 32768, None) == 4   # block count overflows


def test_mmq_bf16_validation(lib):
    f = lib.q4k_mmq_bf16
    assert f(P, P, P, None, 4, 64, 256, None) == 1      # no output
    assert f(None, P, P, P, 4, 64, 256, None) == 1
    assert f(P, P, P, P + 1, 4, 64, 256, None) == 3     # bf16 output needs 2 bytes
    assert f(P, P, P, P, 4, 64, 300, None) == 2         # k not a multiple of 256
    assert f(P, P, P, P, 0, 64, 256, None) == 2


def test_ffn_noalloc_validation(lib):
    f = lib.ffn_swiglu_q4k_noalloc
    # the same argument checks as ffn_swiglu_q4k, without a workspace
    assert f(None, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 0, P, None) == 1
    assert f(P, P, P, 1, P, 0, 1, 300, 768, None, None, 0, 0, P, None) == 2
    assert f(P + 4, P, P, 1, P, 0, 1, 256, 768, None, None, 0, 0, P, None) == 3
    # a layout beyond the fixed scratch (4096 tokens of 5120/17408 need about
    # 390 MB) is refused before any HIP call
    assert lib.ffn_swiglu_q4k_workspace_bytes(4096, 5120, 17408, 0, 0) > B.Q4K_NOALLOC_SCRATCH_BYTES
    assert f(P, P, P, 1, P, 1, 4096, 5120, 17408, None, None, 0, 0, P, None) == 8
    # 512 tokens of the same FFN fit
    assert lib.ffn_swiglu_q4k_workspace_bytes(512, 5120, 17408, 0, 0) <= B.Q4K_NOALLOC_SCRATCH_BYTES


def test_read_hook_validation(lib):
    r = lib.q4k_test_read
    assert r(None, 16, P, None) == 1
    assert r(P, 16, None, None) == 1
    assert r(P, 0, P, None) == 2
    assert r(P, 24, P, None) == 2        # not a multiple of 16
    assert r(P + 8, 16, P, None) == 3
    assert r(P, 16, P + 2, None) == 3


def test_fp8_validation(lib):
    a = lib.fp8_absmax_rows
    assert a(None, 4, 16, P, None) == 1
    assert a(P, 4, 16, None, None) == 1
    assert a(P, 0, 16, P, None) == 2
    assert a(P, 4, 0, P, None) == 2
    assert a(P + 2, 4, 16, P, None) == 3           # f32 rows need 4 bytes
    assert a(P, 4, 16, P + 1, None) == 3
    q = lib.fp8_quantize_rows
    assert q(P, 4, 16, P, None, None) == 1
    assert q(P, 4, -1, P, P, None) == 2
    assert q(P, 4, 16, P + 2, P, None) == 3
    assert q(P, 1 << 30, 1 << 30, P, P, None) == 4  # one value per thread: grid too large
    g = lib.fp8_gemm_dequant
    assert g(P, P, P, P, None, 4, 64, 128, None) == 1
    assert g(None, P, P, P, P, 4, 64, 128, None) == 1
    assert g(P, P, P, P, P, 0, 64, 128, None) == 2
    assert g(P, P, P, P, P, 4, 0, 128, None) == 2
    assert g(P, P, P, P, P, 4, 64, 120, None) == 2    # k not a multiple of 16
    assert g(P, P, P, P, P, 4, 64, 0, None) == 2
    assert g(P, P, P, P, P, 4, 64, (1 << 20) + 16, None) == 2
    assert g(P, P, P, P, P, 64 * 65535 + 1, 64, 128, None) == 2
    assert g(P + 4, P, P, P, P, 4, 64, 128, None) == 3  # codes need 16 bytes
    assert g(P, P, P + 8, P, P, 4, 64, 128, None) == 3
    assert g(P, P + 2, P, P, P, 4, 64, 128, None) == 3
    assert g(P, P, P, P, P + 2, 4, 64, 128, None) == 3
