"""CPU oracle for the weight-only LUT-quantized matmul -- TEST INFRASTRUCTURE.

Plain, slow, obviously correct numpy code, fp64 accumulation. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.
The library under ``weight_only_lut_amd`` never calls it: it has no CPU
fallback, and it shares no code, table or constant with this package.

What it computes (page 2, FLUTE abstract: weight-only quantization with the
dequantization fused into the matmul; page 2, BitMoD abstract: per-group
rescaling of partial sums, which is the same sum in another order):

    W_hat[n, k] = T[c[n, k]] * s[n, k // group]      (s[0] when group == 0)
    y[m, n]     = sum_k x[m, k] * W_hat[n, k]

and, with per-group zero points z (page 1, LogbQuant abstract: asymmetric
linear quantization), W_hat[n, k] = s[n, k // group] * (T[c[n, k]] - z[n, k // group]);
with per-group data types (page 2, BitMoD abstract), T is the table the
group's type id selects; binary-coded weights (page 4, AlphaTuning
abstract) are W_hat[n, k] = sum_i alpha_i[n, g] * (2 bit_i(c[n, k]) - 1).

Every function cites the passage it follows. Parity status of each function
is in the docstring; all are pinned by tests/test_oracle.py, and the
quantizer (``oracle.quantize``: round-to-nearest onto a table, the weight
error, the logarithmic table and its base search) by
tests/test_oracle_quantize.py.
"""

from .lutq_ref import (  # noqa: F401
    pack_codes,
    unpack_codes,
    dequant,
    reference,
    reference_rows,
    dequant_bcq,
    reference_bcq,
    error_bound,
    error_bound_bf16,
    check,
)
from . import quantize  # noqa: F401
