"""GPU parity for per-group zero points (lutq_matmul_zp, and zeros in the
fused launch): W_hat = s * (T[c] - z) against the oracle.

- every path and workgroup shape, with and without K splits, 2/3/4 bits,
  groups of 128 and 256, ragged widths and ragged / sliced batches;
- one-hot activations on every shape: each output is s * (T[c] - z),
  compared bit for bit;
- z = 0 gives bit for bit the launch without zero points;
- asymmetric INT (uniform table 0..2^b-1, zero points inside the range);
- a fused launch mixing matrices with and without zero points equals the
  single-matrix launches bit for bit;
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


def zeros_for(s, T, seed):
    """Zero points inside the table's range, one per group (fp16)."""
    lo, hi = float(T.astype(np.float32).min()), float(T.astype(np.float32).max())
    return np.random.default_rng(seed).uniform(lo, hi, s.shape).astype(np.float16)


def assert_close(y, x, c, T, s, group, z, rows=None):
    if rows is None:
        y_ref, B = oracle.reference(x, c, T, s, group, zeros=z)
        yy = y
    else:
        y_ref, B = oracle.reference_rows(x, c, T, s, group, rows, zeros=z)
        yy = y[:, rows]
    ok, worst = oracle.check(yy, y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table,group", [(4, "nf", 128), (3, "lloyd_max", 256), (2, "int", 128),
                                              (4, "int", 384)])
@pytest.mark.parametrize("M", [1, 5, 16, 45])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_zero_points_every_shape(lutq, path, tiles, bits, table, group, M, ksplit):
    N, K = 293, 768
    c, T, s, x = workloads.small_case(bits, table, group, M, N, K, seed=600 + bits + M)
    z = zeros_for(s, T, 601 + M)
    P = lutq.repack(dev(c), bits, group)
    xd, Td, sd = dev(x), dev(T), dev(s)
    y = lutq.matmul(xd, P, Td, sd, zeros=dev(z), path=path, tiles=tiles, ksplit=ksplit)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), x, c, T, s, group, z)
    # z = 0 is the launch without zero points, bit for bit
    y0 = lutq.matmul(xd, P, Td, sd, zeros=torch.zeros_like(sd), path=path, tiles=tiles,
                     ksplit=ksplit)
    y1 = lutq.matmul(xd, P, Td, sd, path=path, tiles=tiles, ksplit=ksplit)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table", [(2, "int"), (3, "lloyd_max"), (4, "nf")])
def test_zero_points_one_hot_every_shape(lutq, path, tiles, bits, table):
    # one-hot activations: each output is one weight, s * (T[c] - z), with the
    # difference and the product each rounded once in fp32, then to fp16
    N, K = 150, 256
    c, T, s, _ = workloads.small_case(bits, table, 128, 1, N, K, seed=630 + bits)
    z = zeros_for(s, T, 631 + bits)
    x = np.eye(K, dtype=np.float16)
    P = lutq.repack(dev(c), bits, 128)
    y = lutq.matmul(dev(x), P, dev(T), dev(s), zeros=dev(z), path=path, tiles=tiles).cpu().numpy()
    g = np.arange(K) // 128
    d = T[c].astype(np.float32) - z[:, g].astype(np.float32)
    want = (s[:, g].astype(np.float32) * d).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.T.view(np.uint16))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_asymmetric_int(lutq, bits, M):
    # s * (q - z): uniform table 0 .. 2^b - 1, a zero point per group inside it
    N, K = 200, 1024
    L = 1 << bits
    rng = np.random.default_rng(610 + bits)
    q = rng.integers(0, L, (N, K)).astype(np.uint8)
    T = np.arange(L).astype(np.float16)
    s = rng.uniform(0.001, 0.01, (N, K // 128)).astype(np.float16)
    z = rng.uniform(0, L - 1, (N, K // 128)).astype(np.float16)
    x = draw.activations(M, K, (611, M))
    P = lutq.repack(dev(q), bits, 128)
    y = lutq.matmul(dev(x), P, dev(T), dev(s), zeros=dev(z))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), x, q, T, s, 128, z)


@pytest.mark.parametrize("M", [1, 16])
def test_fused_mixed_zero_points(lutq, M):
    K = 512
    mats = []
    for i, N in enumerate((130, 48, 77)):
        c, T, s, _ = workloads.small_case(4, "nf", 128, 1, N, K, seed=620 + i)
        mats.append((c, T, s, zeros_for(s, T, 621 + i) if i != 1 else None))
    x = draw.activations(M, K, (622, M))
    xd = dev(x)
    dm = []
    for c, T, s, z in mats:
        item = (lutq.repack(dev(c), 4, 128), dev(T), dev(s))
        dm.append(item + ((dev(z),) if z is not None else ()))
    for path, tiles in (("gemv", 2), ("mfma", 4), ("mfma", 7)):
        ys = lutq.matmul_multi(xd, dm, path=path, tiles=tiles)
        torch.cuda.synchronize()
        for y, (c, T, s, z), d in zip(ys, mats, dm):
            if z is None:
                y_ref, B = oracle.reference(x, c, T, s, 128)
            else:
                y_ref, B = oracle.reference(x, c, T, s, 128, zeros=z)
            ok, worst = oracle.check(y.cpu().numpy(), y_ref, B)
            assert ok, f"max err/bound = {worst:.3g}"
            y1 = lutq.matmul(xd, d[0], d[1], d[2], zeros=d[3] if len(d) > 3 else None,
                             path=path, tiles=tiles)
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


def test_zero_points_llama_projection(lutq):
    w = workloads.WORKLOADS["nf4_layer"]
    c, T, s = workloads.quantized(w, "gate")
    z = zeros_for(s, T, 630)
    P = lutq.repack(dev(c), w.bits, w.group)
    Td, sd, zd = dev(T), dev(s), dev(z)
    for M in (1, 8, 16, 32):
        x = workloads.activations(w, M, "gate")
        y = lutq.matmul(dev(x), P, Td, sd, zeros=zd).cpu().numpy()
        assert_close(y, x, c, T, s, w.group, z)
