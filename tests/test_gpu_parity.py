"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

- packing: bit-exact round trip, the GPU bytes equal the documented layout
  (tests/layout_spec.py), and code bits above `bits` are masked;
- one-hot activations decode every weight through the whole kernel,
  bit-exactly: y = fp16(fp32(T[c]) * fp32(s));
- random cases for every width, table kind, grouping, batch size (including
  ragged and sliced batches), ragged N, both paths and forced K splits,
  within |y - y_ref| <= 1e-3 * sum|x w| + 1e-5;
- the full-size workloads in the launch configuration the benchmark times,
  every output compared;
- determinism and the degenerate cases (K = 0, M = 0, N = 0, misalignment).
"""

import numpy as np
import pytest

import oracle
from synth import draw, tables, workloads

from . import layout_spec

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


def run(lutq, codes, T, s, x, bits, group, **kw):
    P = lutq.repack(dev(codes), bits, group)
    y = lutq.matmul(dev(x), P, dev(T), dev(s), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_close(y, x, codes, T, s, group, rows=None):
    if rows is None:
        y_ref, B = oracle.reference(x, codes, T, s, group)
        yy = y
    else:
        y_ref, B = oracle.reference_rows(x, codes, T, s, group, rows)
        yy = y[:, rows]
    ok, worst = oracle.check(yy, y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"
    return worst


# -- packing ------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (64, 256), (1000, 1024)])
def test_repack_matches_layout_and_roundtrips(lutq, bits, N, K):
    c = draw.integers((N, K), 1 << bits, (41, bits, N, K))
    P = lutq.repack(dev(c), bits, 128)
    torch.cuda.synchronize()
    got = P.data.cpu().numpy()[: P.nbytes]
    assert np.array_equal(got, layout_spec.encode(c, bits))
    assert np.array_equal(layout_spec.decode(got, N, K, bits), c)
    assert np.array_equal(lutq.unpack(P).cpu().numpy(), c)


@pytest.mark.parametrize("bits", [2, 3])
def test_repack_masks_high_bits(lutq, bits):
    c = draw.integers((20, 256), 256, (42, bits))
    P = lutq.repack(dev(c), bits, 0)
    assert np.array_equal(lutq.unpack(P).cpu().numpy(), c & ((1 << bits) - 1))


# -- one-hot activations: every weight through the full kernel, bit-exact ----

@pytest.mark.parametrize("bits,table", [(4, "nf"), (3, "lloyd_max"), (2, "int"), (4, "log")])
@pytest.mark.parametrize("group", [128, 0])
@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_one_hot_decodes_every_weight(lutq, bits, table, group, path):
    N, K = 40, 256
    c, T, s, _ = workloads.small_case(bits, table, group, 1, N, K, seed=50 + bits)
    x = np.eye(K, dtype=np.float16)
    y = run(lutq, c, T, s, x, bits, group, path=path)
    sk = s[:, np.arange(K) // 128] if group else np.full((N, K), s[0])
    want = (T[c].astype(np.float32) * sk.astype(np.float32)).astype(np.float16)  # [N, K]
    assert np.array_equal(y.view(np.uint16), want.T.view(np.uint16))


# -- random cases ---------------------------------------------------------------

CASES = [
    # bits, table, group, N, K
    (4, "nf", 128, 200, 640),
    (4, "int", 128, 16, 128),
    (3, "lloyd_max", 128, 131, 1024),
    (2, "nf", 128, 64, 384),
    (4, "log", 0, 72, 512),
    (3, "lloyd_max", 256, 48, 768),
    (2, "int", 0, 33, 256),
    (4, "nf", 512, 80, 1024),
    (4, "int", 384, 45, 1152),        # 3 chunks per group
    (3, "lloyd_max", 640, 29, 1280),  # 5 chunks per group
]


@pytest.mark.parametrize("bits,table,group,N,K", CASES)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 9, 16, 31, 32, 33])
@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_parity_random(lutq, bits, table, group, N, K, M, path):
    dist = "laplace" if table == "log" else "student_t"
    kw = {"b": 0.015} if table == "log" else {"nu": 4.0, "scale": 0.02}
    c, T, s, x = workloads.small_case(bits, table, group, M, N, K, seed=N + K + bits,
                                      dist=dist, **kw)
    y = run(lutq, c, T, s, x, bits, group, path=path)
    assert_close(y, x, c, T, s, group)


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table,group", [(4, "nf", 128), (3, "lloyd_max", 0), (2, "int", 256),
                                              (4, "int", 384)])
@pytest.mark.parametrize("M", [1, 5, 16, 32, 45])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_parity_every_shape(lutq, path, tiles, bits, table, group, M, ksplit):
    # 293 rows = 19 tiles: at 8 tiles per wave two full row blocks and a
    # ragged third (3 tiles, the last one 5 rows); 45 batch rows = a full
    # slice plus a ragged one on either path.
    N, K = 293, 768
    c, T, s, x = workloads.small_case(bits, table, group, M, N, K, seed=300 + bits + M)
    y = run(lutq, c, T, s, x, bits, group, path=path, tiles=tiles, ksplit=ksplit)
    assert_close(y, x, c, T, s, group)


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table", [(2, "int"), (3, "lloyd_max"), (4, "nf")])
def test_one_hot_every_shape(lutq, path, tiles, bits, table):
    N, K = 150, 256
    c, T, s, _ = workloads.small_case(bits, table, 128, 1, N, K, seed=60 + bits)
    x = np.eye(K, dtype=np.float16)
    y = run(lutq, c, T, s, x, bits, 128, path=path, tiles=tiles)
    want = (T[c].astype(np.float32) * s[:, np.arange(K) // 128].astype(np.float32)).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.T.view(np.uint16))


@pytest.mark.parametrize("ksplit", [1, 2, 3, 7, 100])
@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_parity_forced_k_splits(lutq, ksplit, path):
    c, T, s, x = workloads.small_case(4, "nf", 128, 4, 150, 1024 + 128, seed=7)
    y = run(lutq, c, T, s, x, 4, 128, path=path, ksplit=ksplit)
    assert_close(y, x, c, T, s, 128)


def test_deterministic(lutq):
    c, T, s, x = workloads.small_case(4, "nf", 128, 8, 1024, 4096, seed=8)
    P = lutq.repack(dev(c), 4, 128)
    xs, Ts, ss = dev(x), dev(T), dev(s)
    for path in ("gemv", "mfma"):
        a = lutq.matmul(xs, P, Ts, ss, path=path).cpu().numpy()
        b = lutq.matmul(xs, P, Ts, ss, path=path).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_lut_permutation_invariance(lutq):
    # permuting the table and remapping the codes leaves y bit-identical
    c, T, s, x = workloads.small_case(4, "nf", 128, 3, 96, 512, seed=12)
    perm = np.random.default_rng(0).permutation(16)
    inv = np.argsort(perm)
    y1 = run(lutq, c, T, s, x, 4, 128)
    y2 = run(lutq, inv[c].astype(np.uint8), T[perm], s, x, 4, 128)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


# -- degenerate cases -----------------------------------------------------------

def test_empty_and_zero_sizes(lutq):
    T = dev(tables.normal_float(4))
    # K = 0: the empty sum
    P = lutq.repack(torch.empty((8, 0), dtype=torch.uint8, device="cuda"), 4, 0)
    y = lutq.matmul(torch.empty((3, 0), dtype=torch.float16, device="cuda"), P, T,
                    dev(np.ones(1, np.float16)), out=torch.full((3, 8), 7.0, dtype=torch.float16,
                                                                 device="cuda"))
    assert torch.all(y == 0)
    # M = 0 and N = 0: nothing to do
    c, Tn, s, x = workloads.small_case(4, "nf", 128, 1, 16, 128, seed=1)
    P = lutq.repack(dev(c), 4, 128)
    y = lutq.matmul(torch.empty((0, 128), dtype=torch.float16, device="cuda"), P, dev(Tn), dev(s))
    assert y.shape == (0, 16)
    P0 = lutq.repack(torch.empty((0, 128), dtype=torch.uint8, device="cuda"), 4, 128)
    y = lutq.matmul(dev(x), P0, dev(Tn), dev(np.ones(1, np.float16)))
    assert y.shape == (1, 0)


def test_misaligned_activations_rejected(lutq):
    c, T, s, x = workloads.small_case(4, "nf", 128, 1, 16, 128, seed=2)
    P = lutq.repack(dev(c), 4, 128)
    big = torch.zeros(129, dtype=torch.float16, device="cuda")
    xm = big[1:].view(1, 128)
    with pytest.raises(lutq.LutqError) as e:
        lutq.matmul(xm, P, dev(T), dev(s))
    assert e.value.code == -4


def test_single_row_and_single_tile(lutq):
    for N in (1, 15, 16, 17):
        c, T, s, x = workloads.small_case(3, "lloyd_max", 128, 2, N, 256, seed=N)
        for path in ("gemv", "mfma"):
            assert_close(run(lutq, c, T, s, x, 3, 128, path=path), x, c, T, s, 128)


# -- full-size workloads ----------------------------------------------------------

def _full(lutq, wname, mat, Ms, paths=("auto",)):
    """Every output of a full-size workload matrix against the oracle."""
    w = workloads.WORKLOADS[wname]
    c, T, s = workloads.quantized(w, mat)
    P = lutq.repack(dev(c), w.bits, w.group)
    Td, sd = dev(T), dev(s)
    worst = 0.0
    for M in Ms:
        x = workloads.activations(w, M, mat)
        xd = dev(x)
        for path in paths:
            y = lutq.matmul(xd, P, Td, sd, path=path).cpu().numpy()
            worst = max(worst, assert_close(y, x, c, T, s, w.group))
    return worst


def test_full_nf4_1k(lutq):
    _full(lutq, "nf4_1k", None, (1,), paths=("auto", "gemv", "mfma"))


def test_full_int4_up_proj(lutq):
    _full(lutq, "int4_up_proj", None, (1,), paths=("auto", "gemv", "mfma"))


@pytest.mark.parametrize("mat", ["sq", "wide"])
def test_full_lm3(lutq, mat):
    _full(lutq, "lm3", mat, (1, 4, 8), paths=("auto", "gemv", "mfma"))


def test_full_log4_70b(lutq):
    # 28672 rows, every output compared: the 7-tile MFMA shape at 8, 16 and
    # 32 batch rows (batch 32 is the configuration the benchmark times)
    _full(lutq, "log4_70b", None, (1, 8, 16, 32))


@pytest.mark.parametrize("mat", ["q", "k", "v", "o", "gate", "up", "down"])
def test_full_nf4_layer(lutq, mat):
    _full(lutq, "nf4_layer", mat, (1, 8, 16, 32))
