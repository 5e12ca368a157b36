"""GPU parity for binary-coded weights (lutq_matmul_bcq): q planes, an alpha
per plane, row and group, W_hat = sum_p alpha_p (2 bit_p(c) - 1), against the
oracle.

- every GEMV and MFMA shape, with and without K splits, q = 2, 3, 4, groups
  of 128 and 256, ragged widths and ragged / sliced batches;
- one-hot activations on every shape and width: each output is one weight,
  sum_p alpha_p (2 bit_p - 1) summed in plane order in fp32, so a plane bit
  read from the wrong position (the GEMV table or the MFMA path's register
  decode) changes it; compared bit for bit;
- power-of-two plane factors against the plain LUT launch of the uniform
  table 2c - (2^q - 1) (both against the oracle, and each other);
- a Llama-3-8B projection (14336 x 4096, the benchmark's binary-coded
  shape) at q = 3 at the benchmark's batch sizes, every output compared.
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


def make(q, N, K, group, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1 << q, (N, K)).astype(np.uint8)
    # AlphaTuning-like factors: each plane about half the previous one
    a = np.stack([rng.uniform(0.01, 0.03, (N, K // group)) / 2 ** p for p in range(q)])
    return c, a.astype(np.float16)


def check(y, x, c, a, group, rows=None):
    y_ref, B = oracle.reference_bcq(x, c, a, group, rows=rows)
    ok, worst = oracle.check(y if rows is None else y[:, rows], y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("q,group", [(2, 128), (3, 256), (4, 128)])
@pytest.mark.parametrize("M", [1, 5, 16, 45])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_bcq_every_shape(lutq, path, tiles, q, group, M, ksplit):
    N, K = 293, 768
    c, a = make(q, N, K, group, 800 + q + M)
    x = draw.activations(M, K, (801, M))
    P = lutq.repack(dev(c), q, group)
    y = lutq.matmul_bcq(dev(x), P, dev(a), path=path, tiles=tiles, ksplit=ksplit)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), x, c, a, group)


@pytest.mark.parametrize("q", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 16])
def test_bcq_power_of_two_planes_match_the_lut_launch(lutq, q, M):
    N, K = 200, 512
    rng = np.random.default_rng(810 + q)
    c = rng.integers(0, 1 << q, (N, K)).astype(np.uint8)
    base = (2.0 ** rng.integers(-9, -5, (N, K // 128))).astype(np.float16)
    a = np.stack([(base.astype(np.float64) * 2 ** p).astype(np.float16) for p in range(q)])
    T = (2 * np.arange(1 << q) - ((1 << q) - 1)).astype(np.float16)
    x = draw.activations(M, K, (811, M))
    P = lutq.repack(dev(c), q, 128)
    y_bcq = lutq.matmul_bcq(dev(x), P, dev(a)).cpu().numpy()
    y_lut = lutq.matmul(dev(x), P, dev(T), dev(base)).cpu().numpy()
    check(y_bcq, x, c, a, 128)
    y_ref, B = oracle.reference(x, c, T, base, 128)
    ok, worst = oracle.check(y_lut, y_ref, B)
    assert ok, worst
    ok, worst = oracle.check(y_bcq, y_lut.astype(np.float64), B)
    assert ok, worst


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("q", [2, 3, 4])
def test_bcq_one_hot_every_shape(lutq, path, tiles, q):
    N, K = 150, 256
    c, a = make(q, N, K, 128, 820 + q)
    x = np.eye(K, dtype=np.float16)
    P = lutq.repack(dev(c), q, 128)
    y = lutq.matmul_bcq(dev(x), P, dev(a), path=path, tiles=tiles).cpu().numpy()
    # y[k, n] = sum over planes, in order, of alpha_p[n][k / 128] * (+-1), in fp32
    g = np.arange(K) // 128
    want = np.zeros((N, K), np.float32)
    for p in range(q):
        sign = (2 * ((c >> p) & 1).astype(np.int32) - 1).astype(np.float32)
        want = want + a[p][:, g].astype(np.float32) * sign
    assert np.array_equal(y.view(np.uint16), want.astype(np.float16).T.view(np.uint16))


def test_bcq_llama_projection(lutq):
    w = workloads.WORKLOADS["nf4_layer"]
    _, m = w.matrix("gate")
    N, K = m.N, m.K
    c, a = make(3, N, K, 128, 830)
    P = lutq.repack(dev(c), 3, 128)
    ad = dev(a)
    for M in (1, 8, 16, 32):
        x = workloads.activations(w, M, "gate")
        y = lutq.matmul_bcq(dev(x), P, ad).cpu().numpy()
        check(y, x, c, a, 128)
