"""GPU parity for per-group data types (lutq_matmul_typed): group g of row n
reads table types[n, g], W_hat = s * (T_type[c] - z), against the oracle.

- every path and workgroup shape, with and without K splits and zero
  points, 1 to 4 tables of 2, 3 and 4 bits, ragged widths and batches;
- one-hot activations on every shape, with and without zero points: each
  output is one weight of its group's table, compared bit for bit;
- one table with all ids 0 gives the plain launch bit for bit;
- ids at or above the table count follow the documented mapping;
- a Llama-3-8B projection with four table kinds, every output compared.
"""

import numpy as np
import pytest

import oracle
from synth import draw, tables, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KINDS = ("nf", "int", "lloyd_max", "log")


@pytest.fixture(scope="module")
def lutq():
    import weight_only_lut_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(bits, ntypes, N, K, group, seed, zeros=False):
    rng = np.random.default_rng(seed)
    luts = np.stack([tables.make(k, bits) for k in KINDS[:ntypes]])
    c = rng.integers(0, 1 << bits, (N, K)).astype(np.uint8)
    types = rng.integers(0, ntypes, (N, K // group)).astype(np.uint8)
    s = rng.uniform(0.005, 0.03, (N, K // group)).astype(np.float16)
    z = rng.uniform(-0.5, 0.5, s.shape).astype(np.float16) if zeros else None
    return c, luts, types, s, z


def check(y, x, c, luts, types, s, z, group, rows=None):
    if rows is None:
        y_ref, B = oracle.reference(x, c, luts, s, group, zeros=z, types=types)
        yy = y
    else:
        y_ref, B = oracle.reference_rows(x, c, luts, s, group, rows, zeros=z, types=types)
        yy = y[:, rows]
    ok, worst = oracle.check(yy, y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("zeros", [False, True])
def test_types_one_hot_every_shape(lutq, path, tiles, bits, zeros):
    # one-hot activations: each output is one weight of its group's table,
    # s * (T_type[c] - z), rounded once in fp32 per step, then to fp16
    N, K = 150, 512
    c, luts, types, s, z = make(bits, 4, N, K, 128, 740 + bits, zeros)
    x = np.eye(K, dtype=np.float16)
    P = lutq.repack(dev(c), bits, 128)
    y = lutq.matmul(dev(x), P, dev(luts), dev(s), types=dev(types),
                    zeros=dev(z) if z is not None else None, path=path, tiles=tiles).cpu().numpy()
    g = np.arange(K) // 128
    w = luts[types[:, g], c].astype(np.float32)
    if z is not None:
        w = w - z[:, g].astype(np.float32)
    want = (s[:, g].astype(np.float32) * w).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.T.view(np.uint16))


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,ntypes,group", [(4, 4, 128), (3, 3, 256), (2, 2, 128), (4, 1, 128),
                                               (3, 4, 384)])
@pytest.mark.parametrize("M", [1, 5, 16, 45])
@pytest.mark.parametrize("ksplit,zeros", [(1, False), (3, True)])
def test_types_every_shape(lutq, path, tiles, bits, ntypes, group, M, ksplit, zeros):
    N, K = 293, 768
    c, luts, types, s, z = make(bits, ntypes, N, K, group, 700 + bits + M, zeros)
    x = draw.activations(M, K, (701, M))
    P = lutq.repack(dev(c), bits, group)
    y = lutq.matmul(dev(x), P, dev(luts), dev(s), types=dev(types),
                    zeros=dev(z) if z is not None else None, path=path, tiles=tiles, ksplit=ksplit)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), x, c, luts, types, s, z, group)


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_one_type_is_the_plain_launch(lutq, path):
    N, K = 150, 512
    c, luts, types, s, _ = make(4, 1, N, K, 128, 710)
    x = draw.activations(7, K, (711,))
    P = lutq.repack(dev(c), 4, 128)
    xd, Ld, sd = dev(x), dev(luts), dev(s)
    y_t = lutq.matmul(xd, P, Ld, sd, types=dev(np.zeros_like(types)), path=path)
    y_p = lutq.matmul(xd, P, Ld[0], sd, path=path)
    assert torch.equal(y_t.view(torch.int16), y_p.view(torch.int16))


def test_out_of_range_type_ids(lutq):
    # an id is taken modulo 4; one (mod 4) at or above the table count reads table 0
    N, K = 64, 256
    c, luts, types, s, _ = make(4, 3, N, K, 128, 720)
    raw = np.random.default_rng(721).integers(0, 256, types.shape).astype(np.uint8)
    eff = (raw % 4).astype(np.uint8)
    eff[eff >= 3] = 0
    x = draw.activations(3, K, (722,))
    P = lutq.repack(dev(c), 4, 128)
    for path in ("gemv", "mfma"):
        y = lutq.matmul(dev(x), P, dev(luts), dev(s), types=dev(raw), path=path).cpu().numpy()
        check(y, x, c, luts, eff, s, None, 128)


def test_types_llama_projection(lutq):
    w = workloads.WORKLOADS["nf4_layer"]
    c, _, s = workloads.quantized(w, "up")
    luts = np.stack([tables.make(k, 4) for k in KINDS])
    types = np.random.default_rng(730).integers(0, 4, s.shape).astype(np.uint8)
    P = lutq.repack(dev(c), 4, w.group)
    Ld, sd, td = dev(luts), dev(s), dev(types)
    for M in (1, 8, 16, 32):
        x = workloads.activations(w, M, "up")
        y = lutq.matmul(dev(x), P, Ld, sd, types=td).cpu().numpy()
        check(y, x, c, luts, types, s, None, w.group)
