"""Seeded synthetic inputs for the weight-only LUT matmul.

This package is the one place both sides of a parity check draw their inputs
from: the HIP path (through the ``weight_only_lut_amd`` binding) and the CPU
oracle (under ``oracle/``). It produces *data* only:

- weight matrices and activations with the distributions of the workloads
  (``draw``),
- the 2^b-entry lookup tables those weights are quantized to (``tables``),
- per-group / per-tensor fp16 scales and round-to-nearest codes (``rtn``),
- the named workloads, sizes and seeds (``workloads``).

It holds none of the matmul's arithmetic: no unpacking of packed bits, no
dequantization and no product. The GPU never quantizes; it receives the
codes, table and scales made here exactly as the oracle does.
"""

from . import draw, tables, rtn, workloads  # noqa: F401
