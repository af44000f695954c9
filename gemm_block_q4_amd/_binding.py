"""ctypes binding of ``libq4k.so`` (the C ABI in ``include/q4k.h``).

Argument marshalling only: every torch tensor is checked for dtype, for
holding at least the bytes the call will touch, for contiguity and for living
on the GPU (``ValueError`` otherwise), then its device pointer and the current
HIP stream are handed to the library, which validates shapes, alignment and
sizes again on the host.  Every computation runs in the library's HIP kernels; there is
no fallback, and a missing library raises :class:`Q4KError`.
"""

from __future__ import annotations

import ctypes
import os

Q4K_F32, Q4K_BF16 = 0, 1
Q4K_REGIME_AUTO, Q4K_REGIME_DECODE, Q4K_REGIME_PREFILL, Q4K_REGIME_DECODE_Q8 = 0, 1, 2, 3
Q4K_DECODE_MAX_TOKENS = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class Q4KError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"q4k status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libq4k.so")


_VP, _SZ, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int

_SIGNATURES = {
    "q4k_weight_bytes": (_SZ, [_I, _I]),
    "q4k_status_string": (ctypes.c_char_p, [_I]),
    "q4k_gemv": (_I, [_VP, _VP, _VP, _I, _I, _I, _VP]),
    "q8_1_quantize": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP]),
    "q4k_mmq": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _VP]),
    "q4k_mmq_bf16": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _VP]),
    "q4k_test_mmq_partials": (_I, [_VP, _VP, _I, _I, _I, _VP, _VP]),
    "q4k_q8_gemv": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _VP]),
    "q4k_quantize": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "q6k_weight_bytes": (_SZ, [_I, _I]),
    "q6k_gemv": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "ffn_swiglu_q4k_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "ffn_swiglu_q4k": (_I, [_VP, _VP, _VP, _I, _VP, _I, _I, _I, _I, _VP, _VP, _I, _I, _VP,
                            _VP, _SZ, _VP]),
    "q4k_test_read": (_I, [_VP, _SZ, _VP, _VP]),
    "ffn_swiglu_q4k_noalloc": (_I, [_VP, _VP, _VP, _I, _VP, _I, _I, _I, _I, _VP, _VP, _I, _I, _VP,
                                    _VP]),
    "fp8_absmax_rows": (_I, [_VP, _I, _I, _VP, _VP]),
    "fp8_quantize_rows": (_I, [_VP, _I, _I, _VP, _VP, _VP]),
    "fp8_gemm_dequant": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _VP]),
}

#: Bytes of the fixed per-device scratch buffer of ffn_swiglu_q4k_noalloc.
Q4K_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def load_library(path: str | None = None, share_torch_runtime: bool = True) -> ctypes.CDLL:
    """Load ``libq4k.so`` once; raise if it has not been built.

    torch is imported first, so that the library's HIP runtime dependency
    binds to the runtime torch already loaded: loaded the other way round, the
    process would hold two HIP runtimes, and the library would not know
    torch's streams or devices.  ``share_torch_runtime=False`` (host-only
    checks of the argument validation) skips that import."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if share_torch_runtime:
        import torch  # noqa: F401
    path = path or library_path()
    if not os.path.exists(path):
        raise Q4KError(-1, f"HIP library not built: {path} is missing "
                           "(run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().q4k_status_string(status).decode()
        raise Q4KError(status, msg)


# dtype names accepted for each kind of buffer (torch dtype names)
_BYTES = ("uint8", "int8")
_F32 = ("float32",)
_BF16 = ("int16", "uint16", "bfloat16")
_I32 = ("int32", "uint32")


def _ptrs(*specs) -> list:
    """Device pointers of the tensors in ``specs``, each ``(tensor, nbytes,
    dtypes, name)``: every tensor is first checked for an accepted dtype (None:
    any), for holding at least ``nbytes`` bytes and for contiguity, then every
    tensor for living on the GPU.  ``None`` passes through (the library reports
    a missing pointer)."""
    for t, nbytes, dtypes, name in specs:
        if t is None:
            continue
        if dtypes is not None and str(t.dtype).replace("torch.", "") not in dtypes:
            raise ValueError(f"{name}: dtype {t.dtype} not one of {', '.join(dtypes)}")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{name}: holds {have} bytes, the call needs {nbytes}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensor must be contiguous")
    for t, _, _, name in specs:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: tensor must live on the GPU")
    return [None if t is None else t.data_ptr() for t, _, _, _ in specs]


def _pos(*v: int) -> bool:
    return all(int(a) > 0 for a in v)


def _x_dtypes(x_dtype: int):
    return _BF16 if x_dtype == Q4K_BF16 else _F32


def _x_size(x_dtype: int) -> int:
    return 2 if x_dtype == Q4K_BF16 else 4


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# -- host helpers ---------------------------------------------------------------

def q4k_weight_bytes(rows: int, cols: int) -> int:
    return int(load_library().q4k_weight_bytes(rows, cols))


def q6k_weight_bytes(rows: int, cols: int) -> int:
    return int(load_library().q6k_weight_bytes(rows, cols))


def ffn_swiglu_q4k_workspace_bytes(m: int, hidden: int, inter: int, top_k: int = 0,
                                   regime: int = Q4K_REGIME_AUTO) -> int:
    return int(load_library().ffn_swiglu_q4k_workspace_bytes(m, hidden, inter, top_k, regime))


# -- device entry points --------------------------------------------------------
# (sizes are only computed for positive shapes; the library rejects the rest)

def _q8_specs(w, qs, ds, m: int, n: int, k: int, ok: bool):
    """Checks of a Q4_K matrix [n, k] and the Q8_1 activations [m, k]."""
    return ((w, q4k_weight_bytes(n, k) if ok else 0, _BYTES, "w"),
            (qs, m * k if ok else 0, _BYTES, "qs"),
            (ds, 4 * m * (k // 32) if ok else 0, _I32, "ds"))


def q4k_gemv(w, x, y, m: int, n: int, k: int, stream=None) -> None:
    """y[m, n] = x[m, k] @ dequant(w)[n, k]^T on the GPU (``q4k_gemv``)."""
    ok = _pos(m, n, k)
    pw, px, py = _ptrs((w, q4k_weight_bytes(n, k) if ok else 0, _BYTES, "w"),
                       (x, 4 * m * k if ok else 0, _F32, "x"),
                       (y, 4 * m * n if ok else 0, _F32, "y"))
    _check(load_library().q4k_gemv(pw, px, py, m, n, k, _stream(stream)))


def q8_1_quantize(x, x_dtype: int, m: int, k: int, qs, ds, stream=None) -> None:
    ok = _pos(m, k)
    px, pq, pd = _ptrs((x, _x_size(x_dtype) * m * k if ok else 0, _x_dtypes(x_dtype), "x"),
                       (qs, m * k if ok else 0, _BYTES, "qs"),
                       (ds, 4 * m * (k // 32) if ok else 0, _I32, "ds"))
    _check(load_library().q8_1_quantize(px, x_dtype, m, k, pq, pd, _stream(stream)))


def q4k_mmq(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    ok = _pos(m, n, k)
    p = _ptrs(*_q8_specs(w, qs, ds, m, n, k, ok), (y, 4 * m * n if ok else 0, _F32, "y"))
    _check(load_library().q4k_mmq(*p, m, n, k, _stream(stream)))


def q4k_mmq_bf16(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    """q4k_mmq with the result stored as bfloat16 bits (y: int16 or uint16 [m, n])."""
    ok = _pos(m, n, k)
    p = _ptrs(*_q8_specs(w, qs, ds, m, n, k, ok), (y, 2 * m * n if ok else 0, _BF16, "y"))
    _check(load_library().q4k_mmq_bf16(*p, m, n, k, _stream(stream)))


def q4k_quantize(x, x_dtype: int, rows: int, cols: int, w, stream=None) -> None:
    """Encode weights x [rows, cols] (f32 or bf16 bits) to block_q4_K bytes w."""
    ok = _pos(rows, cols)
    px, pw = _ptrs((x, _x_size(x_dtype) * rows * cols if ok else 0, _x_dtypes(x_dtype), "x"),
                   (w, q4k_weight_bytes(rows, cols) if ok else 0, _BYTES, "w"))
    _check(load_library().q4k_quantize(px, x_dtype, rows, cols, pw, _stream(stream)))


def q4k_q8_gemv(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    """y[m, n] = reference dot of Q8_1 rows (qs, ds) with the Q4_K rows, m <= 8."""
    ok = _pos(m, n, k)
    p = _ptrs(*_q8_specs(w, qs, ds, m, n, k, ok), (y, 4 * m * n if ok else 0, _F32, "y"))
    _check(load_library().q4k_q8_gemv(*p, m, n, k, _stream(stream)))


def q6k_gemv(w, x, y, n: int, k: int, stream=None) -> None:
    """y[n] = dequant(w)[n, k] @ x[k] for Q6_K weights w (one f32 token)."""
    ok = _pos(n, k)
    pw, px, py = _ptrs((w, q6k_weight_bytes(n, k) if ok else 0, _BYTES, "w"),
                       (x, 4 * k if ok else 0, _F32, "x"),
                       (y, 4 * n if ok else 0, _F32, "y"))
    _check(load_library().q6k_gemv(pw, px, py, n, k, _stream(stream)))


def q4k_test_mmq_partials(w, qs, m: int, n: int, k: int, partials, stream=None) -> None:
    ok = _pos(m, n, k)
    pw, pq, pp = _ptrs((w, q4k_weight_bytes(n, k) if ok else 0, _BYTES, "w"),
                       (qs, m * k if ok else 0, _BYTES, "qs"),
                       (partials, 4 * m * n * (k // 32) if ok else 0, _I32, "partials"))
    _check(load_library().q4k_test_mmq_partials(pw, pq, m, n, k, pp, _stream(stream)))


def ffn_swiglu_q4k(w_gate, w_up, w_down, x, x_dtype: int, m: int, hidden: int, inter: int,
                   y, workspace, n_experts: int = 1, ids=None, wts=None, top_k: int = 0,
                   regime: int = Q4K_REGIME_AUTO, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ok = _pos(m, hidden, inter, n_experts)
    gu = n_experts * q4k_weight_bytes(inter, hidden) if ok else 0
    dn = n_experts * q4k_weight_bytes(hidden, inter) if ok else 0
    pairs = m * top_k if ok and ids is not None and top_k > 0 else 0
    pg, pu, pd, px, pi, pt, py, pws = _ptrs(
        (w_gate, gu, _BYTES, "w_gate"), (w_up, gu, _BYTES, "w_up"), (w_down, dn, _BYTES, "w_down"),
        (x, _x_size(x_dtype) * m * hidden if ok else 0, _x_dtypes(x_dtype), "x"),
        (ids, 4 * pairs, _I32, "ids"), (wts, 4 * pairs, _F32, "wts"),
        (y, 4 * m * hidden if ok else 0, _F32, "y"), (workspace, 0, None, "workspace"))
    _check(load_library().ffn_swiglu_q4k(pg, pu, pd, n_experts, px, x_dtype, m, hidden, inter, pi, pt,
                                         top_k, regime, py, pws, ws_bytes, _stream(stream)))


def ffn_swiglu_q4k_noalloc(w_gate, w_up, w_down, x, x_dtype: int, m: int, hidden: int, inter: int,
                           y, n_experts: int = 1, ids=None, wts=None, top_k: int = 0,
                           regime: int = Q4K_REGIME_AUTO, stream=None) -> None:
    """ffn_swiglu_q4k on the library's fixed scratch buffer (no workspace)."""
    ok = _pos(m, hidden, inter, n_experts)
    gu = n_experts * q4k_weight_bytes(inter, hidden) if ok else 0
    dn = n_experts * q4k_weight_bytes(hidden, inter) if ok else 0
    pairs = m * top_k if ok and ids is not None and top_k > 0 else 0
    pg, pu, pd, px, pi, pt, py = _ptrs(
        (w_gate, gu, _BYTES, "w_gate"), (w_up, gu, _BYTES, "w_up"), (w_down, dn, _BYTES, "w_down"),
        (x, _x_size(x_dtype) * m * hidden if ok else 0, _x_dtypes(x_dtype), "x"),
        (ids, 4 * pairs, _I32, "ids"), (wts, 4 * pairs, _F32, "wts"),
        (y, 4 * m * hidden if ok else 0, _F32, "y"))
    _check(load_library().ffn_swiglu_q4k_noalloc(pg, pu, pd, n_experts, px, x_dtype, m, hidden, inter,
                                                 pi, pt, top_k, regime, py, _stream(stream)))


def q4k_test_read(buf, nbytes: int, sink, stream=None) -> None:
    """Plain read of the first ``nbytes`` bytes of ``buf`` (read-ceiling hook)."""
    pb, ps = _ptrs((buf, nbytes, None, "buf"), (sink, 4, _I32, "sink"))
    _check(load_library().q4k_test_read(pb, nbytes, ps, _stream(stream)))


# -- per-row FP8 (E4M3) recipe ---------------------------------------------------

def fp8_absmax_rows(x, rows: int, cols: int, absmax, stream=None) -> None:
    """absmax[rows] = max |x[r, :]| of an f32 matrix."""
    ok = _pos(rows, cols)
    px, pa = _ptrs((x, 4 * rows * cols if ok else 0, _F32, "x"),
                   (absmax, 4 * rows if ok else 0, _F32, "absmax"))
    _check(load_library().fp8_absmax_rows(px, rows, cols, pa, _stream(stream)))


def fp8_quantize_rows(x, rows: int, cols: int, absmax, q, stream=None) -> None:
    """q[rows, cols] = E4M3 codes of x times 448/absmax of its row."""
    ok = _pos(rows, cols)
    px, pa, pq = _ptrs((x, 4 * rows * cols if ok else 0, _F32, "x"),
                       (absmax, 4 * rows if ok else 0, _F32, "absmax"),
                       (q, rows * cols if ok else 0, _BYTES, "q"))
    _check(load_library().fp8_quantize_rows(px, rows, cols, pa, pq, _stream(stream)))


def fp8_gemm_dequant(a, a_absmax, w, w_absmax, y, m: int, n: int, k: int, stream=None) -> None:
    """y[m, n] = bf16(A_fp8 @ W_fp8^T) * (a_absmax/448) * (w_absmax/448)."""
    ok = _pos(m, n, k)
    p = _ptrs((a, m * k if ok else 0, _BYTES, "a"), (a_absmax, 4 * m if ok else 0, _F32, "a_absmax"),
              (w, n * k if ok else 0, _BYTES, "w"), (w_absmax, 4 * n if ok else 0, _F32, "w_absmax"),
              (y, 4 * m * n if ok else 0, _F32, "y"))
    _check(load_library().fp8_gemm_dequant(*p, m, n, k, _stream(stream)))
