"""Pins for the CPU oracle: each check rests on something other than the oracle.

- packing: hand-derived byte fixtures and an exhaustive round trip;
- dequantization: the uniform table reproduces INT RTN (an integer formula);
- product: exact rational arithmetic on tiny non-square shapes, linearity in
  the scale, one-hot activations;
- acceptance: the tolerance accepts and rejects where it should;
- mutations: plausible mistakes planted in a copy of the oracle fail a pin.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import lutq_ref
from synth import draw, rtn, tables, workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows


# -- packing ------------------------------------------------------------------

def test_pack_matches_hand_derived_bytes():
    for bits, codes, want in _read_fixture("pack_lsb_first.txt"):
        b = int(bits)
        c = np.array([[int(v) for v in codes.split()]], dtype=np.uint8)
        got = oracle.pack_codes(c, b)[0]
        assert bytes(got) == bytes(int(h, 16) for h in want.split()), (bits, codes)
        assert np.array_equal(oracle.unpack_codes(got[None], 1, c.shape[1], b), c)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip_every_value_every_offset(bits):
    # every code value at every bit offset within a 96-bit period
    period = 96 // bits
    L = 1 << bits
    rows = []
    for v in range(L):
        for off in range(period):
            r = np.zeros(period + 3, np.uint8)
            r[off] = v
            rows.append(r)
            r2 = np.full(period + 3, L - 1, np.uint8)
            r2[off] = v
            rows.append(r2)
    c = np.stack(rows)
    p = oracle.pack_codes(c, bits)
    assert p.shape[1] == (c.shape[1] * bits + 7) // 8
    assert np.array_equal(oracle.unpack_codes(p, c.shape[0], c.shape[1], bits), c)


@pytest.mark.parametrize("bits,table", [(2, "nf"), (3, "lloyd_max"), (4, "int"), (4, "log")])
def test_quantize_pack_unpack_roundtrip(bits, table):
    c, T, s, _ = workloads.small_case(bits, table, 128, 1, 37, 384, seed=bits)
    p = oracle.pack_codes(c, bits)
    assert np.array_equal(oracle.unpack_codes(p, *c.shape, bits), c)
    assert c.max() < (1 << bits)


def test_pack_rejects_out_of_range_codes():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.array([[8]], np.uint8), 3)


# -- dequantization -----------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("group", [128, 0])
def test_uniform_lut_reproduces_int_rtn(bits, group):
    """A uniform table T[i] = i - z dequantizes exactly like asymmetric INT RTN."""
    W = draw.weights("normal_outliers", 48, 512, (7, bits, group), sigma=0.02, p=0.01, mult=10.0)
    T = tables.int_uniform(bits)
    z = 1 << (bits - 1)
    c, s = rtn.quantize(W, T, group, "int")
    # textbook asymmetric INT RTN, written with integers: q = clamp(rint(w/s) + z, 0, 2^b - 1)
    s64 = (np.repeat(s.astype(np.float64), group, axis=1) if group else np.full(W.shape, float(s[0])))
    r = W.astype(np.float64) / s64
    assert not np.any(np.abs(r - np.floor(r) - 0.5) < 1e-12), "exact tie in test data"
    q = np.clip(np.rint(r) + z, 0, (1 << bits) - 1).astype(np.int64)
    assert np.array_equal(q, c.astype(np.int64))
    int_deq = (q - z).astype(np.float32) * s64.astype(np.float32)
    assert np.array_equal(oracle.dequant(c, T, s, group).view(np.uint32), int_deq.view(np.uint32))


def test_dequant_scale_index_is_along_k():
    # a hand case: N=2, K=256, group=128, every code 1 -> T[1]
    T = np.array([0, 1, 2, 3], np.float16)
    c = np.ones((2, 256), np.uint8)
    s = np.array([[2, 3], [5, 7]], np.float16)
    w = oracle.dequant(c, T, s, 128)
    assert np.all(w[0, :128] == 2) and np.all(w[0, 128:] == 3)
    assert np.all(w[1, :128] == 5) and np.all(w[1, 128:] == 7)


# -- the product --------------------------------------------------------------

def _exact(x, codes, T, s, group):
    """sum_k x*T[c]*s in exact rationals; the fp32 product T*s is rounded as IEEE does."""
    M, K = x.shape
    N = codes.shape[0]
    w = np.empty((N, K), dtype=object)
    for n in range(N):
        for k in range(K):
            sv = s.reshape(-1)[0] if group == 0 else s[n, k // group]
            # T and s are fp16, so their exact product has <= 22 significant bits
            # and needs one rounding to fp32: do it through Fraction -> float32
            prod = Fraction(float(T[codes[n, k]])) * Fraction(float(sv))
            w[n, k] = Fraction(float(np.float32(float(prod))))
    y = [[sum(Fraction(float(x[m, k])) * w[n, k] for k in range(K)) for n in range(N)]
         for m in range(M)]
    return y


@pytest.mark.parametrize("bits,table,group,M,N,K", [
    (4, "nf", 128, 3, 5, 256),
    (3, "lloyd_max", 128, 2, 3, 384),
    (2, "nf", 0, 1, 4, 128),
    (4, "log", 0, 3, 2, 256),
])
def test_product_matches_exact_rationals(bits, table, group, M, N, K):
    c, T, s, x = workloads.small_case(bits, table, group, M, N, K, seed=11 + bits)
    y, B = oracle.reference(x, c, T, s, group)
    ex = _exact(x, c, T, s, group)
    for m in range(M):
        for n in range(N):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-12 * B[m, n] + 1e-300


def test_product_is_linear_in_the_scale():
    c, T, s, x = workloads.small_case(4, "nf", 128, 4, 33, 512, seed=3)
    y1, _ = oracle.reference(x, c, T, s, 128)
    y2, _ = oracle.reference(x, c, T, (s.astype(np.float32) * 4).astype(np.float16), 128)
    assert np.array_equal(y2, 4 * y1)


def test_one_hot_activation_decodes_single_weights():
    c, T, s, _ = workloads.small_case(3, "lloyd_max", 128, 1, 9, 256, seed=5)
    x = np.eye(256, dtype=np.float16)[[0, 1, 127, 128, 255]]
    y, _ = oracle.reference(x, c, T, s, 128)
    for m, k in enumerate([0, 1, 127, 128, 255]):
        want = T[c[:, k]].astype(np.float32) * s[:, k // 128].astype(np.float32)
        assert np.array_equal(y[m], want.astype(np.float64))


def test_reference_rows_agrees_with_reference():
    c, T, s, x = workloads.small_case(4, "int", 128, 3, 40, 256, seed=9)
    y, B = oracle.reference(x, c, T, s, 128)
    rows = np.array([0, 7, 39, 13])
    yr, Br = oracle.reference_rows(x, c, T, s, 128, rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(Br, B[:, rows])


# -- acceptance ---------------------------------------------------------------

def test_check_accepts_inside_and_rejects_outside_the_bound():
    c, T, s, x = workloads.small_case(4, "nf", 128, 2, 16, 256, seed=2)
    y, B = oracle.reference(x, c, T, s, 128)
    bound = oracle.error_bound(B)
    assert oracle.check(y + 0.9 * bound, y, B)[0]
    bad = y.copy()
    bad[1, 3] += 1.5 * bound[1, 3]
    ok, worst = oracle.check(bad, y, B)
    assert not ok and worst > 1.0
    nan = y.copy()
    nan[0, 0] = np.nan
    assert not oracle.check(nan, y, B)[0]


# -- planted mistakes: each must fail one of the pins above -------------------

def _mutant_dequant(kind):
    original = lutq_ref.dequant

    def f(codes, lut, scales, group, zeros=None, types=None):
        N, K = codes.shape
        t = lut.astype(np.float32)[codes]
        if kind == "group_by_row":
            s = scales.astype(np.float32).reshape(-1)[(np.arange(N) // max(group, 1)) % scales.size]
            return t * s[:, None]
        if kind == "sign":
            return -original(codes, lut, scales, group)
        if kind == "scale_dropped":
            return t
        raise AssertionError(kind)
    return f


@pytest.mark.parametrize("kind", ["group_by_row", "sign", "scale_dropped"])
def test_planted_dequant_mistakes_are_caught(monkeypatch, kind):
    c, T, s, x = workloads.small_case(4, "nf", 128, 2, 3, 256, seed=21)
    ex = _exact(x, c, T, s, 128)
    monkeypatch.setattr(lutq_ref, "dequant", _mutant_dequant(kind))
    y, B = oracle.reference(x, c, T, s, 128)
    err = max(abs(y[m, n] - float(ex[m][n])) for m in range(2) for n in range(3))
    assert err > 1e-6


def test_planted_transpose_is_caught():
    c, T, s, x = workloads.small_case(4, "nf", 0, 2, 2, 128, seed=22)
    ex = _exact(x, c, T, s, 0)
    y, _ = oracle.reference(x, c, T, s, 0)
    assert max(abs(y.T[m, n] - float(ex[m][n])) for m in range(2) for n in range(2)) > 1e-6


# -- zero points (W_hat = s * (T[c] - z) per group) ---------------------------

def _zp_case(seed, M=3, N=4, K=256, bits=4, table="nf"):
    c, T, s, x = workloads.small_case(bits, table, 128, M, N, K, seed=seed)
    z = np.random.default_rng(seed).uniform(-0.6, 0.6, s.shape).astype(np.float16)
    return c, T, s, z, x


def _exact_zp(x, c, T, s, z, group):
    M, K = x.shape
    N = c.shape[0]
    return [[sum(Fraction(float(x[m, k])) * Fraction(float(s[n, k // group]))
                 * (Fraction(float(T[c[n, k]])) - Fraction(float(z[n, k // group])))
                 for k in range(K)) for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("bits,table,group,K", [(4, "nf", 128, 256), (3, "lloyd_max", 256, 512),
                                                (2, "int", 128, 384)])
def test_zero_points_match_exact_rationals(bits, table, group, K):
    c, T, s, x = workloads.small_case(bits, table, group, 2, 3, K, seed=31 + bits)
    z = np.random.default_rng(bits).uniform(-0.6, 0.6, s.shape).astype(np.float16)
    y, B = oracle.reference(x, c, T, s, group, zeros=z)
    ex = _exact_zp(x, c, T, s, z, group)
    for m in range(2):
        for n in range(3):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-12 * B[m, n] + 1e-300


def test_zero_points_shift_invariance():
    # T + d and z + d give the same weights (all values exact in fp16)
    rng = np.random.default_rng(32)
    T = (np.arange(16) - 8).astype(np.float16)
    c = rng.integers(0, 16, (5, 256)).astype(np.uint8)
    s = (2.0 ** rng.integers(-8, -3, (5, 2))).astype(np.float16)
    z = (rng.integers(-16, 17, (5, 2)) / 4).astype(np.float16)
    x = rng.normal(0, 1, (3, 256)).astype(np.float16)
    d = np.float16(2.5)
    y1, _ = oracle.reference(x, c, T, s, 128, zeros=z)
    y2, _ = oracle.reference(x, c, (T + d).astype(np.float16), s, 128, zeros=(z + d).astype(np.float16))
    assert np.array_equal(y1, y2)


def test_zero_points_are_integer_asymmetric_rtn():
    # uniform table T[i] = i with an integer zero point per group is
    # asymmetric INT dequantization s * (q - z); integer x and power-of-two
    # scales make the whole product exact
    rng = np.random.default_rng(33)
    for bits in (2, 3, 4):
        L = 1 << bits
        T = np.arange(L).astype(np.float16)
        q = rng.integers(0, L, (6, 384)).astype(np.uint8)
        z = rng.integers(0, L, (6, 3))
        e = rng.integers(-6, 0, (6, 3))
        x = rng.integers(-8, 9, (4, 384))
        y, _ = oracle.reference(x.astype(np.float16), q, T, (2.0 ** e).astype(np.float16), 128,
                                zeros=z.astype(np.float16))
        want = np.zeros((4, 6))
        for g in range(3):
            blk = slice(128 * g, 128 * (g + 1))
            iw = q[:, blk].astype(np.int64) - z[:, g:g + 1]          # [6, 128] integers
            want += (x[:, blk].astype(np.int64) @ iw.T) * (2.0 ** e[:, g])[None, :]
        assert np.array_equal(y, want)


def test_zero_points_zero_is_the_plain_product():
    c, T, s, z, x = _zp_case(34)
    y0, _ = oracle.reference(x, c, T, s, 128)
    yz, _ = oracle.reference(x, c, T, s, 128, zeros=np.zeros_like(s))
    assert np.allclose(yz, y0, rtol=1e-6, atol=1e-9)
    with pytest.raises(ValueError):
        oracle.dequant(c, T, s[:, :1], 0, zeros=s[:, :1])


def _mutant_zp(kind):
    def f(codes, lut, scales, group, zeros=None, types=None):
        N, K = codes.shape
        g = K // group
        t = lut.astype(np.float64)[codes].reshape(N, g, group)
        sc = scales.astype(np.float64).reshape(N, g, 1)
        z = zeros.astype(np.float64).reshape(N, g, 1)
        if kind == "sign":
            return (sc * (t + z)).reshape(N, K)
        if kind == "by_row":
            return (sc * (t - zeros.astype(np.float64).T.reshape(-1)[:N * g].reshape(N, g, 1))).reshape(N, K)
        if kind == "unscaled":
            return (sc * t - z).reshape(N, K)
        raise AssertionError(kind)
    return f


@pytest.mark.parametrize("kind", ["sign", "by_row", "unscaled"])
def test_planted_zero_point_mistakes_are_caught(monkeypatch, kind):
    c, T, s, z, x = _zp_case(35, M=2, N=3, K=256)
    ex = _exact_zp(x, c, T, s, z, 128)
    monkeypatch.setattr(lutq_ref, "dequant", _mutant_zp(kind))
    y, _ = oracle.reference(x, c, T, s, 128, zeros=z)
    err = max(abs(y[m, n] - float(ex[m][n])) for m in range(2) for n in range(3))
    assert err > 1e-6


# -- per-group data types (a table per type id) --------------------------------

def _typed_case(seed, M=2, N=3, K=256, bits=3, ntypes=3, with_zeros=False):
    rng = np.random.default_rng(seed)
    L = 1 << bits
    luts = np.stack([tables.make(k, bits) for k in ("nf", "int", "lloyd_max", "nf")[:ntypes]])
    luts[-1] = (luts[-1].astype(np.float32) * 0.5).astype(np.float16)   # distinct tables
    c = rng.integers(0, L, (N, K)).astype(np.uint8)
    types = rng.integers(0, ntypes, (N, K // 128)).astype(np.uint8)
    s = rng.uniform(0.01, 0.05, (N, K // 128)).astype(np.float16)
    z = rng.uniform(-0.5, 0.5, s.shape).astype(np.float16) if with_zeros else None
    x = rng.normal(0, 1, (M, K)).astype(np.float16)
    return c, luts, types, s, z, x


def _exact_typed(x, c, luts, types, s, z, group):
    M, K = x.shape
    N = c.shape[0]
    zf = (lambda n, g: Fraction(float(z[n, g]))) if z is not None else (lambda n, g: Fraction(0))
    return [[sum(Fraction(float(x[m, k])) * Fraction(float(s[n, k // group]))
                 * (Fraction(float(luts[types[n, k // group], c[n, k]])) - zf(n, k // group))
                 for k in range(K)) for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("with_zeros", [False, True])
def test_data_types_match_exact_rationals(with_zeros):
    c, luts, types, s, z, x = _typed_case(41, with_zeros=with_zeros)
    y, B = oracle.reference(x, c, luts, s, 128, zeros=z, types=types)
    ex = _exact_typed(x, c, luts, types, s, z, 128)
    for m in range(2):
        for n in range(3):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-12 * B[m, n] + 1e-300


def test_data_types_relabelling_invariance():
    # the same tables under other ids, the ids mapped along: same weights
    c, luts, types, s, z, x = _typed_case(42, N=6, K=512, ntypes=4)
    perm = np.array([2, 0, 3, 1])
    inv = np.argsort(perm)
    y1, _ = oracle.reference(x, c, luts, s, 128, types=types)
    y2, _ = oracle.reference(x, c, luts[perm], s, 128, types=inv[types].astype(np.uint8))
    assert np.array_equal(y1, y2)


def test_data_types_single_type_is_the_plain_product():
    c, luts, types, s, z, x = _typed_case(43, N=5, K=384)
    y_typed, _ = oracle.reference(x, c, luts[1:2], s, 128, types=np.zeros_like(types))
    y_plain, _ = oracle.reference(x, c, luts[1], s, 128)
    assert np.allclose(y_typed, y_plain, rtol=1e-6, atol=1e-9)


def test_planted_type_index_by_row_is_caught(monkeypatch):
    c, luts, types, s, z, x = _typed_case(44)
    ex = _exact_typed(x, c, luts, types, s, z, 128)

    def by_row(codes, lut, scales, group, zeros=None, types=None):
        N, K = codes.shape
        ty = np.repeat(types.T.reshape(-1)[:N * (K // group)].reshape(N, K // group), group, 1)
        t = lut.astype(np.float64)[ty, codes]
        return np.repeat(scales.astype(np.float64), group, 1) * t

    monkeypatch.setattr(lutq_ref, "dequant", by_row)
    y, _ = oracle.reference(x, c, luts, s, 128, types=types)
    assert max(abs(y[m, n] - float(ex[m][n])) for m in range(2) for n in range(3)) > 1e-6


# -- binary-coding quantization ----------------------------------------------

def _bcq_case(seed, q=3, M=2, N=3, K=256, group=128):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1 << q, (N, K)).astype(np.uint8)
    a = rng.uniform(0.001, 0.05, (q, N, K // group)).astype(np.float16)
    x = rng.normal(0, 1, (M, K)).astype(np.float16)
    return c, a, x


def _exact_bcq(x, c, a, group):
    q = a.shape[0]
    M, K = x.shape
    N = c.shape[0]
    return [[sum(Fraction(float(x[m, k])) * sum(
        Fraction(float(a[i, n, k // group])) * (1 if (int(c[n, k]) >> i) & 1 else -1)
        for i in range(q)) for k in range(K)) for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("q,group", [(2, 128), (3, 256), (4, 128)])
def test_bcq_matches_exact_rationals(q, group):
    c, a, x = _bcq_case(50 + q, q=q, K=512, group=group)
    y, B = oracle.reference_bcq(x, c, a, group)
    ex = _exact_bcq(x, c, a, group)
    for m in range(2):
        for n in range(3):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-12 * B[m, n] + 1e-300


def test_bcq_one_plane_is_signed_binary():
    rng = np.random.default_rng(51)
    bits = rng.integers(0, 2, (4, 256)).astype(np.uint8)
    a = rng.uniform(0.01, 0.1, (1, 4, 2)).astype(np.float16)
    w = oracle.dequant_bcq(bits, a, 128)
    sign = np.where(bits == 1, 1.0, -1.0)
    assert np.array_equal(w, sign * np.repeat(a[0].astype(np.float64), 128, axis=1))


@pytest.mark.parametrize("q", [2, 3, 4])
def test_bcq_power_of_two_planes_are_a_uniform_table(q):
    # alpha_i = a 2^i: W_hat = a (2c - (2^q - 1)), the uniform LUT with scale a
    rng = np.random.default_rng(52 + q)
    N, K = 5, 384
    c = rng.integers(0, 1 << q, (N, K)).astype(np.uint8)
    base = (2.0 ** rng.integers(-9, -4, (N, K // 128))).astype(np.float16)
    a = np.stack([(base.astype(np.float64) * 2 ** i).astype(np.float16) for i in range(q)])
    x = rng.normal(0, 1, (3, K)).astype(np.float16)
    T = (2 * np.arange(1 << q) - ((1 << q) - 1)).astype(np.float16)
    y_bcq, _ = oracle.reference_bcq(x, c, a, 128)
    y_lut, _ = oracle.reference(x, c, T, base, 128)
    assert np.array_equal(y_bcq, y_lut)


def test_bcq_equals_a_table_per_group():
    # the 2^q-entry table of each (row, group), indexed by the code
    c, a, x = _bcq_case(53, q=3, N=4, K=384)
    w = oracle.dequant_bcq(c, a, 128)
    for n in range(4):
        for g in range(3):
            table = [sum(float(a[i, n, g]) * (1 if (code >> i) & 1 else -1) for i in range(3))
                     for code in range(8)]
            blk = c[n, 128 * g:128 * (g + 1)]
            assert np.array_equal(w[n, 128 * g:128 * (g + 1)], np.array(table)[blk])


@pytest.mark.parametrize("kind", ["plane_order", "sign", "group_by_row"])
def test_planted_bcq_mistakes_are_caught(monkeypatch, kind):
    c, a, x = _bcq_case(54, q=3, K=256)
    ex = _exact_bcq(x, c, a, 128)
    real = lutq_ref.dequant_bcq
    if kind == "plane_order":
        bad = lambda cc, aa, g: real(cc, aa[::-1], g)
    elif kind == "sign":
        bad = lambda cc, aa, g: real((~cc) & 7, aa, g)
    else:
        bad = lambda cc, aa, g: real(cc, aa.transpose(0, 2, 1).reshape(aa.shape), g)
    monkeypatch.setattr(lutq_ref, "dequant_bcq", bad)
    y, _ = oracle.reference_bcq(x, c, a, 128)
    assert max(abs(y[m, n] - float(ex[m][n])) for m in range(2) for n in range(3)) > 1e-6


# -- bf16 outputs ------------------------------------------------------------

def _to_bf16(v):
    """fp64 -> the nearest bf16 value (ties to even), as fp64; exact via the fp32 bits."""
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_bf16_bound_covers_output_rounding_only():
    # the exact product rounded once to bf16 passes; two bf16 steps off fails
    c, T, s, x = workloads.small_case(4, "nf", 128, 3, 40, 512, seed=60)
    y, B = oracle.reference(x, c, T, s, 128)
    yb = _to_bf16(y)
    assert oracle.check(yb, y, B, out="bf16")[0]
    big = np.abs(y) > 50 * oracle.error_bound(B)       # where rounding dominates the bound
    bad = yb.copy()
    bad[big] = bad[big] * (1 + 2 * 2.0 ** -7)
    assert not oracle.check(bad, y, B, out="bf16")[0]
