"""MI355X (gfx950) Q4_K SwiGLU feed-forward library: Python binding.

The compute lives in ``libq4k.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/q4k.h``).  This package only marshals torch tensors to
device pointers and streams; it has no compute path of its own.  The shared
library is loaded lazily on first use and a missing library raises an error.
"""

from ._binding import (  # noqa: F401
    Q4K_BF16,
    Q4K_F32,
    Q4K_REGIME_AUTO,
    Q4K_REGIME_DECODE,
    Q4K_REGIME_PREFILL,
    Q4K_REGIME_DECODE_Q8,
    Q4K_NOALLOC_SCRATCH_BYTES,
    Q4KError,
    ffn_swiglu_q4k,
    ffn_swiglu_q4k_noalloc,
    ffn_swiglu_q4k_workspace_bytes,
    fp8_absmax_rows,
    fp8_gemm_dequant,
    fp8_quantize_rows,
    library_path,
    load_library,
    q4k_gemv,
    q4k_mmq,
    q4k_mmq_bf16,
    q4k_q8_gemv,
    q4k_quantize,
    q4k_test_mmq_partials,
    q4k_test_read,
    q4k_weight_bytes,
    q6k_gemv,
    q6k_weight_bytes,
    q8_1_quantize,
)
