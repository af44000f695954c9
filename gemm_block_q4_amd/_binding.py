"""ctypes binding of ``libq4k.so`` (the C ABI in ``include/q4k.h``).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity, then their device pointers and the current HIP stream are handed
to the library.  Every computation runs in the library's HIP kernels; there is
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
}


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load ``libq4k.so`` once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
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


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


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

def q4k_gemv(w, x, y, m: int, n: int, k: int, stream=None) -> None:
    """y[m, n] = x[m, k] @ dequant(w)[n, k]^T on the GPU (``q4k_gemv``)."""
    _check(load_library().q4k_gemv(_ptr(w), _ptr(x), _ptr(y), m, n, k, _stream(stream)))


def q8_1_quantize(x, x_dtype: int, m: int, k: int, qs, ds, stream=None) -> None:
    _check(load_library().q8_1_quantize(_ptr(x), x_dtype, m, k, _ptr(qs), _ptr(ds),
                                        _stream(stream)))


def q4k_mmq(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    _check(load_library().q4k_mmq(_ptr(w), _ptr(qs), _ptr(ds), _ptr(y), m, n, k,
                                  _stream(stream)))


def q4k_mmq_bf16(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    """q4k_mmq with the result stored as bfloat16 bits (y: int16 or uint16 [m, n])."""
    _check(load_library().q4k_mmq_bf16(_ptr(w), _ptr(qs), _ptr(ds), _ptr(y), m, n, k,
                                       _stream(stream)))


def q4k_quantize(x, x_dtype: int, rows: int, cols: int, w, stream=None) -> None:
    """Encode weights x [rows, cols] (f32 or bf16 bits) to block_q4_K bytes w."""
    _check(load_library().q4k_quantize(_ptr(x), x_dtype, rows, cols, _ptr(w), _stream(stream)))


def q4k_q8_gemv(w, qs, ds, y, m: int, n: int, k: int, stream=None) -> None:
    """y[m, n] = reference dot of Q8_1 rows (qs, ds) with the Q4_K rows, m <= 8."""
    _check(load_library().q4k_q8_gemv(_ptr(w), _ptr(qs), _ptr(ds), _ptr(y), m, n, k,
                                      _stream(stream)))


def q6k_gemv(w, x, y, n: int, k: int, stream=None) -> None:
    """y[n] = dequant(w)[n, k] @ x[k] for Q6_K weights w (one f32 token)."""
    _check(load_library().q6k_gemv(_ptr(w), _ptr(x), _ptr(y), n, k, _stream(stream)))


def q4k_test_mmq_partials(w, qs, m: int, n: int, k: int, partials, stream=None) -> None:
    _check(load_library().q4k_test_mmq_partials(_ptr(w), _ptr(qs), m, n, k, _ptr(partials),
                                                _stream(stream)))


def ffn_swiglu_q4k(w_gate, w_up, w_down, x, x_dtype: int, m: int, hidden: int, inter: int,
                   y, workspace, n_experts: int = 1, ids=None, wts=None, top_k: int = 0,
                   regime: int = Q4K_REGIME_AUTO, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().ffn_swiglu_q4k(
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), n_experts, _ptr(x), x_dtype, m, hidden, inter,
        _ptr(ids), _ptr(wts), top_k, regime, _ptr(y), _ptr(workspace), ws_bytes,
        _stream(stream)))
