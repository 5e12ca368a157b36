"""GPU parity for the quantizer (lutq_quantize, lutq_quant_error,
lutq_log_base_search) against oracle/quantize.py.

Codes and scales are integers decided by fp64 arithmetic on both sides (the
quotient w / s, the fp64 scale rounded once to fp16), so they must agree bit
for bit; the weight error is a sum in a different order, compared to 1e-9
relative. Cases: every table kind and width, both scale rules, grouped and
tensor-wise scales, ragged row counts, crafted exact ties and fp16 rounding
ties, all-zero and clamped groups, the full-size matrices of the headline and
Llama-70B workloads, and quantize -> repack -> matmul end to end.
"""

import numpy as np
import pytest

import oracle
from oracle import quantize as Q
from synth import draw, tables, workloads

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


def gpu_quantize(lutq, w, T, bits, group, rule):
    c, s = lutq.quantize(dev(w), dev(T), bits, group, rule)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def assert_same(w, T, bits, group, rule, lutq):
    c, s = gpu_quantize(lutq, w, T, bits, group, rule)
    c_ref, s_ref = Q.quantize(w, T, group, rule)
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16)), "scales differ"
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}"


TABLE_CASES = [
    # kind, bits, rule, kwargs
    ("int", 4, "range", {}), ("int", 3, "range", {}), ("int", 2, "range", {}),
    ("int", 4, "absmax", {}), ("nf", 4, "absmax", {}), ("nf", 3, "absmax", {}),
    ("nf", 2, "absmax", {}), ("lloyd_max", 3, "absmax", {}), ("lloyd_max", 4, "absmax", {}),
    ("log", 4, "absmax", {"base": 2 ** 0.5}), ("log", 3, "absmax", {"base": 1.7}),
]


@pytest.mark.parametrize("kind,bits,rule,kw", TABLE_CASES)
@pytest.mark.parametrize("group", [128, 256, 0])
@pytest.mark.parametrize("N,K", [(37, 256), (200, 1024)])
def test_quantize_matches_oracle(lutq, kind, bits, rule, kw, group, N, K):
    if group and K % group:
        pytest.skip("group does not divide K")
    T = tables.make(kind, bits, **kw)
    w = draw.weights("student_t", N, K, (71, bits, N, K, group), nu=4.0, scale=0.02)
    assert_same(w, T, bits, group, rule, lutq)


@pytest.mark.parametrize("group,K", [(512, 1536), (1024, 2048), (384, 1536), (2048, 4096)])
@pytest.mark.parametrize("kind,bits,rule", [("nf", 4, "absmax"), ("int", 3, "range"),
                                            ("log", 2, "absmax")])
def test_quantize_group_sizes(lutq, group, K, kind, bits, rule):
    # every way a group is laid over lanes: 32 or 64 lanes held in registers,
    # or groups that are read twice (not 2^k * 128, or wider than a wave)
    T = tables.make(kind, bits, **({"base": 1.5} if kind == "log" else {}))
    w = draw.weights("student_t", 45, K, (79, group, K, bits), nu=4.0, scale=0.02)
    assert_same(w, T, bits, group, rule, lutq)
    got = lutq.quant_error(dev(w), dev(T), bits, group, rule)
    c, s_ = Q.quantize(w, T, group, rule)
    want = Q.sq_error(w, T, c, s_, group)
    assert abs(got - want) <= 1e-9 * want


TIE_TABLES = [("nf", 4, {}), ("log", 4, {"base": 2 ** 0.5}), ("log", 3, {"base": 1.7}),
              ("lloyd_max", 3, {})]


@pytest.mark.parametrize("kind,bits,kw", TIE_TABLES)
def test_quantize_exact_ties_and_scale_edges(lutq, kind, bits, kw):
    # Log tables sort in an order other than their codes' (positive codes
    # descend), so half of their ties go to the upper entry.
    rng = np.random.default_rng(72)
    T = tables.make(kind, bits, **kw)
    Ts = np.sort(T.astype(np.float64))
    amax = np.abs(Ts).max()
    mids = (Ts[:-1] + Ts[1:]) / 2
    N, K = 8, 512
    L1 = mids.size
    w = np.zeros((N, K), np.float32)
    for n in range(N):
        for g in range(K // 128):
            blk = w[n, g * 128:(g + 1) * 128]
            s = 2.0 ** -(n + 3)                  # exact fp16 scale: absmax = s * amax
            assert np.all(np.float32(mids * s) == mids * s)
            blk[0] = s * amax
            blk[1:1 + L1] = (mids * s).astype(np.float32)               # every midpoint: ties
            blk[1 + L1:1 + 2 * L1] = np.nextafter(mids * s, np.inf).astype(np.float32)
            blk[1 + 2 * L1:] = (rng.normal(0, 0.4, 127 - 2 * L1) * s).astype(np.float32)
    w[0, 256:384] = 0.0                                       # all-zero group -> scale 1
    w[1, 256] = 1e6                                           # clamps to 65504
    w[2, 384:512] = 0.0
    w[2, 384] = np.float32((1 + 2 ** -11) * amax)              # fp16 tie in the scale -> even
    w[3, 384:512] = 0.0
    w[3, 384] = -np.float32((1 + 3 * 2 ** -11) * amax)
    assert_same(w, T, bits, 128, "absmax", lutq)
    Ti = tables.make("int", bits)
    assert_same(w, Ti, bits, 128, "range", lutq)
    assert_same(w, Ti, bits, 0, "range", lutq)


def test_quantize_subnormal_weights_and_scales(lutq):
    # A table with a midpoint at exactly 0: the sign of fp32 subnormal
    # weights and of signed zeros decides their codes (+0 and -0 tie there).
    T = np.array([-1.5, -0.5, 0.5, 1.5], np.float16)
    sub = np.float32(2.0 ** -149)
    rng = np.random.default_rng(78)
    w = np.zeros((4, 256), np.float32)
    w[0, :128] = sub * rng.integers(-40, 41, 128).astype(np.float32)  # subnormals only: scale 1
    w[0, :4] = [sub, -sub, 0.0, -0.0]
    w[1] = rng.normal(0, 1e-6, 256).astype(np.float32)                # fp16-subnormal scales
    w[2] = rng.normal(0, 1e-7, 256).astype(np.float32)
    w[2, 5] = np.float32(3e-5)
    w[3, :128] = rng.normal(0, 1, 128).astype(np.float32)             # subnormals beside normals
    w[3, 10:20] = sub * np.arange(-5, 5, dtype=np.float32)
    for bits_t, rule in ((T, "absmax"), (T, "range")):
        assert_same(w, bits_t, 2, 128, rule, lutq)
        assert_same(w, bits_t, 2, 0, rule, lutq)


@pytest.mark.parametrize("group", [128, 0])
def test_quant_error_matches_oracle(lutq, group):
    T = tables.make("lloyd_max", 3)
    w = draw.weights("laplace", 96, 1024, (73, group), b=0.015)
    got = lutq.quant_error(dev(w), dev(T), 3, group, "absmax")
    c, s = Q.quantize(w, T, group, "absmax")
    want = Q.sq_error(w, T, c, s, group)
    assert abs(got - want) <= 1e-9 * want
    again = lutq.quant_error(dev(w), dev(T), 3, group, "absmax")
    assert again == got                                       # fixed summation order


def test_log_base_search_matches_oracle(lutq):
    w = draw.weights("laplace", 64, 1024, (74,), b=0.015)
    bases = [1.2, 1.35, 2 ** 0.5, 1.6, 2.0, 2.5]
    best, errs = lutq.log_base_search(dev(w), 4, 0, bases)
    best_ref, errs_ref = Q.log_base_search(w, 4, 0, bases)
    assert best == best_ref
    for a, b in zip(errs, errs_ref):
        assert abs(a - b) <= 1e-9 * b


def test_quantize_full_size_headline(lutq):
    w_ = workloads.WORKLOADS["int4_up_proj"]
    w = workloads.weights(w_)
    T = workloads.lut(w_)
    c, s = gpu_quantize(lutq, w, T, 4, 128, "range")
    s_ref = Q.scales(w, T, 128, "range")
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    rows = np.r_[0:64, 7000:7064, w.shape[0] - 64:w.shape[0]]
    c_ref = Q.codes(w[rows], T, s_ref[rows], 128)
    assert np.array_equal(c[rows], c_ref)


def test_quantize_full_size_tensor_wise(lutq):
    w_ = workloads.WORKLOADS["log4_70b"]
    w = workloads.weights(w_)
    T = workloads.lut(w_)
    c, s = gpu_quantize(lutq, w, T, 4, 0, "absmax")
    s_ref = Q.scales(w, T, 0, "absmax")
    assert s.view(np.uint16)[0] == s_ref.view(np.uint16)[0]
    rows = np.r_[0:32, 20000:20032]
    c_ref = Q.codes(w[rows], T, s_ref, 0)
    assert np.array_equal(c[rows], c_ref)


def test_quantize_repack_matmul_end_to_end(lutq):
    T = tables.make("nf", 4)
    w = draw.weights("normal", 300, 1024, (75,), sigma=0.02)
    x = draw.activations(5, 1024, (76,))
    cd, sd = lutq.quantize(dev(w), dev(T), 4, 128, "absmax")
    P = lutq.repack(cd, 4, 128)
    y = lutq.matmul(dev(x), P, dev(T), sd).cpu().numpy()
    c_ref, s_ref = Q.quantize(w, T, 128, "absmax")
    y_ref, B = oracle.reference(x, c_ref, T, s_ref, 128)
    ok, worst = oracle.check(y, y_ref, B)
    assert ok, f"max err/bound = {worst:.3g}"


def _to_16bit(w, dtype):
    """fp32 weights -> torch fp16 / bf16 tensor on the GPU, and the exact fp32 values."""
    t = torch.from_numpy(np.ascontiguousarray(w)).to(dtype)
    return t.cuda(), t.float().numpy()


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("kind,bits,rule,group", [("nf", 4, "absmax", 128), ("int", 3, "range", 0),
                                                   ("log", 4, "absmax", 256), ("int", 2, "range", 512)])
def test_quantize_16bit_weights(lutq, dtype, kind, bits, rule, group):
    # weights as models ship them: widened to fp32 exactly on the GPU
    T = tables.make(kind, bits, **({"base": 2 ** 0.5} if kind == "log" else {}))
    w = draw.weights("student_t", 77, 1024, (76, bits, group), nu=4.0, scale=0.02)
    wd, wv = _to_16bit(w, getattr(torch, dtype))
    c, s = lutq.quantize(wd, dev(T), bits, group, rule)
    torch.cuda.synchronize()
    c_ref, s_ref = Q.quantize(wv, T, group, rule)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c.cpu().numpy(), c_ref)
    got = lutq.quant_error(wd, dev(T), bits, group, rule)
    want = Q.sq_error(wv, T, c_ref, s_ref, group)
    assert abs(got - want) <= 1e-9 * want


def test_log_base_search_fp16_weights(lutq):
    w = draw.weights("laplace", 64, 1024, (78,), b=0.015)
    wd, wv = _to_16bit(w, torch.float16)
    bases = [1.3, 2 ** 0.5, 1.7, 2.2]
    best, errs = lutq.log_base_search(wd, 4, 128, bases)
    best_ref, errs_ref = Q.log_base_search(wv, 4, 128, bases)
    assert best == best_ref
    for a, b in zip(errs, errs_ref):
        assert abs(a - b) <= 1e-9 * b


@pytest.mark.parametrize("kind,bits,rule,group,dtype", [
    ("nf", 4, "absmax", 128, "float32"), ("nf", 3, "absmax", 0, "float32"),
    ("int", 4, "range", 256, "float16"), ("lloyd_max", 3, "absmax", 128, "bfloat16"),
    ("nf", 2, "absmax", 384, "float32")])
def test_tune_table_matches_oracle(lutq, kind, bits, rule, group, dtype):
    # The sums are fp64 in a different order on each side, so a tuned entry
    # could differ only if its centroid fell within ~1e-16 of an fp16
    # rounding boundary; the tables and scales are compared bit for bit.
    T0 = tables.make(kind, bits)
    w = draw.weights("student_t", 90, 1536, (80, bits, group), nu=4.0, scale=0.02)
    wd, wv = _to_16bit(w, getattr(torch, dtype)) if dtype != "float32" else (dev(w), w)
    T, s, errs = lutq.tune_table(wd, dev(T0), bits, group, rule, iters=6)
    T_ref, s_ref, errs_ref = Q.tune_table(wv, T0, group, rule, 6)
    assert np.array_equal(T.cpu().numpy().view(np.uint16), T_ref.view(np.uint16))
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    assert len(errs) == len(errs_ref)
    for a, b in zip(errs, errs_ref):
        assert abs(a - b) <= 1e-9 * b
    assert errs[-1] <= errs[0]
