"""GPU parity for bf16 activations and outputs (lutq_options_t.dtype = bf16).

The kernel scales each (batch row, 128-weight chunk) of x by a power of two
into fp16 range, runs the fp16 arithmetic, and scales back; y is bf16. Bar:
the fp16 bound plus one bf16 rounding (oracle.error_bound_bf16).

- every path and workgroup shape, with and without K splits, grouped and
  tensor-wise scales, ragged widths and batches;
- activations far outside fp16's range (1e-30 .. 1e30, mixed within a chunk
  and across chunks and rows);
- fused launches in bf16 equal the single launches bit for bit;
- a Llama-3-8B projection at the benchmark's batch sizes, every output
  compared.
"""

import numpy as np
import pytest

import oracle
from synth import draw, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lutq():
    import weight_only_lut_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16(v):
    """fp32 values -> (bf16 bits rounded to nearest even, their exact fp32 values)."""
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    bits = (((f + 0x7FFF + ((f >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def from_bf16(t):
    return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def check(y, xv, c, T, s, group, rows=None):
    if rows is None:
        y_ref, B = oracle.reference(xv, c, T, s, group)
        yy = y
    else:
        y_ref, B = oracle.reference_rows(xv, c, T, s, group, rows)
        yy = y[:, rows]
    ok, worst = oracle.check(yy, y_ref, B, out="bf16")
    assert ok, f"max err/bound = {worst:.3g}"


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table,group", [(4, "nf", 128), (3, "lloyd_max", 0), (2, "int", 256)])
@pytest.mark.parametrize("M", [1, 5, 16, 45])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_bf16_every_shape(lutq, path, tiles, bits, table, group, M, ksplit):
    N, K = 293, 768
    c, T, s, _ = workloads.small_case(bits, table, group, 1, N, K, seed=900 + bits + M)
    xb, xv = bf16(draw.activations(M, K, (901, M)).astype(np.float32))
    P = lutq.repack(dev(c), bits, group)
    y = lutq.matmul(dev_bf16(xb), P, dev(T), dev(s), path=path, tiles=tiles, ksplit=ksplit)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    check(from_bf16(y), xv, c, T, s, group)


@pytest.mark.parametrize("path", ["gemv", "mfma"])
@pytest.mark.parametrize("group", [128, 0])
def test_bf16_range_beyond_fp16(lutq, path, group):
    N, K, M = 150, 1024, 6
    c, T, s, _ = workloads.small_case(4, "nf", group, 1, N, K, seed=910)
    rng = np.random.default_rng(911)
    x = rng.normal(0, 1, (M, K)).astype(np.float32)
    x[0] *= 1e30                                   # a huge row
    x[1] *= 1e-30                                  # a tiny row
    x[2, :128] *= 1e20                             # chunks of very different size
    x[2, 128:256] *= 1e-20
    x[3, ::7] *= 1e4                               # mixed within chunks
    x[3, 3::7] *= 1e-4
    x[4, 256:384] = 0.0                            # an all-zero chunk
    x[5] = rng.normal(0, 1e-38, K)                 # bf16 subnormals
    xb, xv = bf16(x)
    P = lutq.repack(dev(c), 4, group)
    y = from_bf16(lutq.matmul(dev_bf16(xb), P, dev(T), dev(s), path=path))
    assert np.all(np.isfinite(y))
    check(y, xv, c, T, s, group)


@pytest.mark.parametrize("M", [1, 16])
def test_bf16_fused_equals_single(lutq, M):
    K = 512
    mats = [workloads.small_case(4, "nf", 128, 1, N, K, seed=920 + i)[:3] for i, N in enumerate((100, 37, 64))]
    xb, xv = bf16(draw.activations(M, K, (921, M)).astype(np.float32))
    xd = dev_bf16(xb)
    dm = [(lutq.repack(dev(c), 4, 128), dev(T), dev(s)) for c, T, s in mats]
    for path, tiles in (("gemv", 1), ("mfma", 2), ("mfma", 7)):
        ys = lutq.matmul_multi(xd, dm, path=path, tiles=tiles)
        for y, (c, T, s), d in zip(ys, mats, dm):
            check(from_bf16(y), xv, c, T, s, 128)
            y1 = lutq.matmul(xd, d[0], d[1], d[2], path=path, tiles=tiles)
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


def test_bf16_llama_projection(lutq):
    w = workloads.WORKLOADS["nf4_layer"]
    c, T, s = workloads.quantized(w, "down")
    P = lutq.repack(dev(c), w.bits, w.group)
    Td, sd = dev(T), dev(s)
    for M in (1, 8, 16, 32):
        xb, xv = bf16(workloads.activations(w, M, "down").astype(np.float32))
        y = from_bf16(lutq.matmul(dev_bf16(xb), P, Td, sd))
        check(y, xv, c, T, s, w.group)
