"""lutq: weight-only LUT-quantized matmul for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of
``liblutq.so`` (declared in ``include/lutq.h``); this package is a thin
ctypes binding with the same names. PyTorch supplies device memory and the
current stream only. There is no CPU fallback: if the library is missing or
no GPU is present, the calls raise.
"""

from ._lib import (  # noqa: F401
    LutqError,
    Packed,
    PATH_AUTO,
    PATH_GEMV,
    PATH_MFMA,
    RULE_ABSMAX,
    RULE_RANGE,
    library_path,
    load_library,
    log_base_search,
    MAX_FUSED,
    MAX_TYPES,
    matmul,
    matmul_bcq,
    matmul_multi,
    matmul_noalloc,
    packed_bytes,
    peak_empty,
    peak_lds,
    peak_mfma,
    peak_stream,
    peak_stream_sink_bytes,
    PEAK_MFMA_16X16X32,
    PEAK_MFMA_32X32X16,
    PEAK_MFMA_FLOPS_PER_ROUND,
    plan,
    quant_error,
    quantize,
    repack,
    strerror,
    tune_table,
    unpack,
)
