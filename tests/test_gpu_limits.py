"""GPU parity at the size limits of the C ABI: K = 2^20 codes per row
(LUTQ_MAX_K) and N close to 2^24 rows (LUTQ_MAX_N).

- K = 2^20 over 40 rows (two whole tiles and a ragged half tile): 4-bit NF
  and 3-bit Lloyd-Max with groups of 128, 2-bit INT with one scale per
  tensor, batch 1, 5 and 32, on the automatic plan and on each path (each
  splits K 85 or 128 ways): every output against the oracle. One-hot
  activations at the first and the last k of the row: each output is one
  weight, compared bit for bit. Zero points, four data types, binary coding
  (q = 3), bf16 activations and a fused launch of two matrices at the same
  K, batch 1 and 32, against the oracle. The quantizer at the same K
  (groups of 128, one scale per tensor, one group per row): codes and scales
  bit for bit.
- N = 2^24 - 5 rows of K = 128 (the last tile ragged), 4-bit: one-hot
  activations at eight positions of the chunk, every one of the 16.8 M
  outputs per row compared bit for bit; random activations at batch 1 and
  32 against the oracle on the first and last tiles and 4096 random rows.
- At both limits, unpack(repack(c)) == c.
  The codes repeat with a prime period of 65521 rows (generating 2 GiB of
  random bytes would dominate the test); the scales do not repeat, so an
  output read from the wrong row still fails.
"""

import numpy as np
import pytest

import oracle
from synth import draw, tables

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_K = 1 << 20
MAX_N = 1 << 24


@pytest.fixture(scope="module")
def lutq():
    import weight_only_lut_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def one_hot_want(c, T, s, group, ks):
    """y[m, n] for x = e_{ks[m]}: fp16(fp32(s[n, k / group]) * fp32(T[c[n, k]]))."""
    out = []
    for k in ks:
        sc = s.reshape(-1)[0] if group == 0 else s[:, k // group]
        out.append((T[c[:, k]].astype(np.float32) * sc.astype(np.float32)).astype(np.float16))
    return np.stack(out)


@pytest.fixture(scope="module", params=[(4, "nf", 128), (3, "lloyd_max", 128), (2, "int", 0)],
                ids=["4bit-g128", "3bit-g128", "2bit-tensor"])
def longest_k(lutq, request):
    bits, table, group = request.param
    N, K = 40, MAX_K
    rng = np.random.default_rng(900 + bits)
    c = rng.integers(0, 1 << bits, (N, K), dtype=np.uint8)
    T = tables.make(table, bits)
    shape = (1,) if group == 0 else (N, K // group)
    s = rng.uniform(0.005, 0.03, shape).astype(np.float16)
    P = lutq.repack(dev(c), bits, group)
    return bits, group, c, T, s, P, dev(T), dev(s)


@pytest.mark.parametrize("M", [1, 5, 32])
@pytest.mark.parametrize("path", [None, "gemv", "mfma"])
def test_longest_k(lutq, longest_k, M, path):
    bits, group, c, T, s, P, Td, sd = longest_k
    K = c.shape[1]
    x = draw.activations(M, K, (910, bits, M))
    kw = {} if path is None else {"path": path}
    plan = lutq.plan(M, c.shape[0], K, bits, **kw)
    assert plan["ksplit"] > 1          # the limit case runs through the K split
    y = lutq.matmul(dev(x), P, Td, sd, **kw).cpu().numpy()
    y_ref, B = oracle.reference(x, c, T, s, group)
    ok, worst = oracle.check(y, y_ref, B)
    assert ok, f"{plan}: max err/bound = {worst:.3g}"


@pytest.mark.parametrize("path", [None, "gemv", "mfma"])
def test_longest_k_one_hot(lutq, longest_k, path):
    bits, group, c, T, s, P, Td, sd = longest_k
    K = c.shape[1]
    ks = [0, 1, K // 2 + 77, K - 2, K - 1]
    x = np.zeros((len(ks), K), np.float16)
    x[np.arange(len(ks)), ks] = 1
    kw = {} if path is None else {"path": path}
    y = lutq.matmul(dev(x), P, Td, sd, **kw).cpu().numpy()
    want = one_hot_want(c, T, s, group, ks)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.fixture(scope="module")
def most_rows(lutq):
    N, K, bits, group = MAX_N - 5, 128, 4, 128
    rng = np.random.default_rng(920)
    c = np.resize(rng.integers(0, 16, (65521, K), dtype=np.uint8), (N, K))
    T = tables.make("nf", bits)
    s = rng.uniform(0.005, 0.03, (N, 1)).astype(np.float16)
    cd = dev(c)
    P = lutq.repack(cd, bits, group)
    del cd
    torch.cuda.synchronize()
    return c, T, s, P, dev(T), dev(s)


@pytest.mark.parametrize("path", [None, "gemv", "mfma"])
def test_most_rows_one_hot(lutq, most_rows, path):
    c, T, s, P, Td, sd = most_rows
    ks = [0, 17, 38, 63, 64, 90, 111, 127]
    x = np.zeros((len(ks), 128), np.float16)
    x[np.arange(len(ks)), ks] = 1
    kw = {} if path is None else {"path": path}
    y = lutq.matmul(dev(x), P, Td, sd, **kw).cpu().numpy()
    want = one_hot_want(c, T, s, 128, ks)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M", [1, 32])
def test_most_rows_random(lutq, most_rows, M):
    c, T, s, P, Td, sd = most_rows
    N = c.shape[0]
    x = draw.activations(M, 128, (921, M))
    y = lutq.matmul(dev(x), P, Td, sd).cpu().numpy()
    rng = np.random.default_rng(922)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 27, N),
                                     rng.integers(0, N, 4096)]))
    y_ref, B = oracle.reference_rows(x, c, T, s, 128, rows)
    ok, worst = oracle.check(y[:, rows], y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"


def _bf16(v):
    """fp32 values -> (bf16 bits rounded to nearest even, their exact fp32 values)."""
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    bits = (((f + 0x7FFF + ((f >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("M", [1, 32])
@pytest.mark.parametrize("variant", ["zeros", "types", "bcq", "bf16", "fused"])
def test_longest_k_variants(lutq, variant, M):
    # every variant at K = 2^20 on the automatic plan (split 85 or 128 ways)
    N, K, group = 40, MAX_K, 128
    rng = np.random.default_rng(930)
    x = draw.activations(M, K, (931, M))
    c = rng.integers(0, 16, (N, K), dtype=np.uint8)
    T = tables.make("nf", 4)
    s = rng.uniform(0.005, 0.03, (N, K // group)).astype(np.float16)
    out = "fp16"
    if variant == "bcq":
        q = 3
        c = c & 7
        a = np.stack([rng.uniform(0.01, 0.03, (N, K // group)) / 2 ** p
                      for p in range(q)]).astype(np.float16)
        y = lutq.matmul_bcq(dev(x), lutq.repack(dev(c), q, group), dev(a)).cpu().numpy()
        results = [(y, oracle.reference_bcq(x, c, a, group))]
    elif variant == "zeros":
        z = rng.uniform(float(T.min()), float(T.max()), s.shape).astype(np.float16)
        y = lutq.matmul(dev(x), lutq.repack(dev(c), 4, group), dev(T), dev(s),
                        zeros=dev(z)).cpu().numpy()
        results = [(y, oracle.reference(x, c, T, s, group, zeros=z))]
    elif variant == "types":
        luts = np.stack([tables.make(k, 4) for k in ("nf", "int", "lloyd_max", "log")])
        ty = rng.integers(0, 4, s.shape).astype(np.uint8)
        y = lutq.matmul(dev(x), lutq.repack(dev(c), 4, group), dev(luts), dev(s),
                        types=dev(ty)).cpu().numpy()
        results = [(y, oracle.reference(x, c, luts, s, group, types=ty))]
    elif variant == "bf16":
        xb, xv = _bf16(x.astype(np.float32) * 1e4)
        xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        yt = lutq.matmul(xd, lutq.repack(dev(c), 4, group), dev(T), dev(s))
        y = (yt.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        results = [(y, oracle.reference(xv, c, T, s, group))]
        out = "bf16"
    else:
        # two matrices sharing x, the second with zero points, in one launch
        N2 = 24
        c2 = rng.integers(0, 16, (N2, K), dtype=np.uint8)
        s2 = rng.uniform(0.005, 0.03, (N2, K // group)).astype(np.float16)
        z2 = rng.uniform(-0.5, 0.5, s2.shape).astype(np.float16)
        Td = dev(T)
        ys = lutq.matmul_multi(dev(x), [(lutq.repack(dev(c), 4, group), Td, dev(s)),
                                        (lutq.repack(dev(c2), 4, group), Td, dev(s2), dev(z2))])
        results = [(ys[0].cpu().numpy(), oracle.reference(x, c, T, s, group)),
                   (ys[1].cpu().numpy(), oracle.reference(x, c2, T, s2, group, zeros=z2))]
    for y, (y_ref, B) in results:
        ok, worst = oracle.check(y, y_ref, B, out=out)
        assert ok, f"{variant}: max err/bound = {worst:.3g}"


@pytest.mark.parametrize("kind,bits,rule,group", [("nf", 4, "absmax", 128), ("int", 4, "range", 128),
                                                  ("nf", 4, "absmax", 0), ("int", 3, "range", MAX_K)])
def test_quantizer_longest_k(lutq, kind, bits, rule, group):
    # the quantizer at K = 2^20: groups of 128, one scale per tensor (three
    # launches), and one group spanning the whole row (read twice); codes and
    # scales bit for bit, the weight error to 1e-9 relative
    from oracle import quantize as Q
    N, K = 40, MAX_K
    w = draw.weights("normal", N, K, (940,), sigma=0.02)
    T = tables.make(kind, bits)
    wd, Td = dev(w), dev(T)
    c, s = lutq.quantize(wd, Td, bits, group, rule)
    c_ref, s_ref = Q.quantize(w, T, group, rule)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16)), "scales differ"
    bad = np.argwhere(c.cpu().numpy() != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}"
    err = lutq.quant_error(wd, Td, bits, group, rule)
    want = Q.sq_error(w, T, c_ref, s_ref, group)
    assert abs(err - want) <= 1e-9 * want


def test_longest_k_unpack(lutq, longest_k):
    # the layout round trip at K = 2^20 (3-bit: the 2-bit and 1-bit planes)
    bits, group, c, T, s, P, Td, sd = longest_k
    assert np.array_equal(lutq.unpack(P).cpu().numpy(), c)


def test_most_rows_unpack(lutq, most_rows):
    c, T, s, P, Td, sd = most_rows
    assert np.array_equal(lutq.unpack(P).cpu().numpy(), c)
