"""Pins for the input generators: tables, scales and RTN codes.

Each table is checked against a property that does not reuse its own
construction: closed forms, symmetry, the defining quantile relation through
an independent normal CDF (math.erf), the Lloyd-Max optimality conditions and
Max's published 1960 levels; RTN is checked against an exact brute-force
argmin in rational arithmetic.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from synth import draw, rtn, tables, workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi_cdf(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _phi_pdf(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def _inv_cdf_bisect(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_int_table_closed_form(bits):
    T = tables.int_uniform(bits)
    assert T.dtype == np.float16
    assert [float(v) for v in T] == list(range(-(1 << (bits - 1)), 1 << (bits - 1)))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_normal_float_quantile_relation(bits):
    L = 1 << bits
    T = tables.normal_float(bits)
    assert np.array_equal(T, -T[::-1])            # symmetric, bit for bit
    assert T[0] == -1 and T[-1] == 1               # scaled to [-1, 1]
    assert np.all(np.diff(T.astype(np.float64)) > 0)
    c = _inv_cdf_bisect((L - 0.5) / L)             # independent inverse CDF
    for i in range(L):
        # T[i] * c is the (i + 1/2)/L quantile of N(0,1); fp16 rounding moves T by <= 2^-11 |T|
        q = _inv_cdf_bisect((i + 0.5) / L) / c
        assert abs(float(T[i]) - q) <= abs(q) * 2.0 ** -11 + 1e-12


def _read_max_table():
    out = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                L, lv, mse = [p.strip() for p in line.split("|")]
                out[int(L)] = ([float(v) for v in lv.split()], float(mse))
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_matches_max_1960_and_is_a_fixed_point(bits):
    L = 1 << bits
    T = tables.lloyd_max_fp64(bits)
    levels, mse_pub = _read_max_table()[L]
    assert np.allclose(T[L // 2:], levels, atol=6e-4, rtol=0)
    assert np.allclose(T, -T[::-1], atol=1e-12)
    # optimality: thresholds are midpoints, levels are conditional means
    t = [(T[j] + T[j + 1]) / 2 for j in range(L - 1)]
    lo = [-math.inf] + t
    hi = t + [math.inf]
    mse = 0.0
    for j in range(L):
        a, b = lo[j], hi[j]
        pa = 0.0 if a == -math.inf else _phi_pdf(a)
        pb = 0.0 if b == math.inf else _phi_pdf(b)
        ca = 0.0 if a == -math.inf else _phi_cdf(a)
        cb = 1.0 if b == math.inf else _phi_cdf(b)
        assert abs((pa - pb) / (cb - ca) - T[j]) < 1e-10
        # E[(X - T_j)^2 ; cell] with E[X^2; cell] = (cb-ca) + a*pa - b*pb
        ex2 = (cb - ca) + (0.0 if a == -math.inf else a * pa) - (0.0 if b == math.inf else b * pb)
        mse += ex2 - 2 * T[j] * (pa - pb) + T[j] ** 2 * (cb - ca)
    assert abs(mse - mse_pub) / mse_pub < 1e-3
    assert np.array_equal(tables.lloyd_max(bits), T.astype(np.float16))


def test_log_table_closed_form():
    T = tables.log_table(4, math.sqrt(2.0))
    for k in range(8):
        if k % 2 == 0:
            assert float(T[k]) == 2.0 ** (-k // 2)          # even exponent: exact power of two
        else:
            want = np.float16(2.0 ** (-(k - 1) // 2) / math.sqrt(2.0))
            assert T[k] == want
        assert T[8 + k] == -T[k]                               # sign is the top bit
    assert np.all(T[:8] > 0)


def test_log_table_other_base():
    T = tables.log_table(4, 2.0)
    assert [float(v) for v in T[:8]] == [2.0 ** -k for k in range(8)]


# -- RTN ----------------------------------------------------------------------

def _brute_codes(r, T):
    Tf = [Fraction(float(t)) for t in T]
    out = []
    for v in r.reshape(-1):
        fv = Fraction(float(v))
        d = [abs(fv - t) for t in Tf]
        out.append(min(range(len(Tf)), key=lambda i: (d[i], i)))  # ties -> lower index
    return np.array(out, np.uint8).reshape(r.shape)


@pytest.mark.parametrize("kind,bits", [("int", 4), ("nf", 4), ("lloyd_max", 3), ("log", 4), ("nf", 2)])
def test_nearest_codes_equal_exact_brute_force(kind, bits):
    T = tables.make(kind, bits)
    rng = np.random.default_rng(5)
    Td = np.sort(T.astype(np.float64))
    mids = (Td[:-1] + Td[1:]) / 2
    r = np.concatenate([
        rng.normal(0, 1.5 * float(np.abs(Td).max()), 3000),
        mids,                                   # exact ties
        np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        Td, [Td[0] - 5, Td[-1] + 5, 0.0, -0.0],
    ])
    assert np.array_equal(rtn.nearest_codes(r, T), _brute_codes(r, T))


def test_tie_goes_to_lower_index():
    T = np.array([0.0, 1.0, -1.0, 2.0], np.float16)       # unsorted on purpose
    assert list(rtn.nearest_codes(np.array([0.5, -0.5, 1.5]), T)) == [0, 0, 1]


def test_absmax_scale_maps_the_largest_weight_to_the_outer_level():
    W = draw.weights("student_t", 16, 512, (3, 3, 0), nu=4.0, scale=0.02)
    T = tables.lloyd_max(3)
    s = rtn.scales(W, T, 128, "absmax")
    amax = np.abs(W.reshape(16, 4, 128)).max(-1).astype(np.float64)
    ideal = amax / float(np.abs(T.astype(np.float64)).max())
    assert np.all(np.abs(s - ideal) <= ideal * 2.0 ** -11)


def test_int_scale_covers_the_group_range():
    W = draw.weights("normal_outliers", 32, 1024, (3, 4, 0), sigma=0.02, p=0.01, mult=10.0)
    s = rtn.scales(W, tables.int_uniform(4), 128, "int").astype(np.float64)
    g = W.reshape(32, 8, 128).astype(np.float64)
    slack = 1 + 2.0 ** -10
    assert np.all(g.max(-1) <= 7 * s * slack) and np.all(g.min(-1) >= -8 * s * slack)
    assert np.all((g.max(-1) >= 7 * s / slack) | (g.min(-1) <= -8 * s / slack))


def test_zero_group_gets_unit_scale_and_tensor_scale_shape():
    W = np.zeros((2, 256), np.float32)
    W[1, 200] = 0.5
    s = rtn.scales(W, tables.normal_float(4), 128, "absmax")
    assert s[0, 0] == 1 and s[0, 1] == 1 and s[1, 0] == 1 and s[1, 1] == np.float16(0.5)
    st = rtn.scales(W, tables.normal_float(4), 0, "absmax")
    assert st.shape == (1,) and st[0] == np.float16(0.5)


def test_workload_definitions():
    W = workloads.WORKLOADS
    assert W["int4_up_proj"].matrices[0].N == 14336 and W["int4_up_proj"].matrices[0].K == 4096
    assert W["log4_70b"].group == 0 and W["log4_70b"].batches == (1, 8, 32)
    assert sum(m.N * m.K for m in W["nf4_layer"].matrices) == 218_103_808
    c, T, s = workloads.quantized(W["nf4_1k"])
    assert c.shape == (1024, 1024) and s.shape == (1024, 8) and T.shape == (16,)
    x = workloads.activations(W["nf4_1k"], 1)
    assert x.dtype == np.float16 and x.shape == (1, 1024)
    # seeded: the same case twice is identical
    c2, _, s2 = workloads.quantized(W["nf4_1k"])
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_outlier_rate():
    W = draw.weights("normal_outliers", 256, 4096, (9, 0, 0), sigma=0.02, p=1e-3, mult=10.0)
    frac = np.mean(np.abs(np.abs(W) - 0.2) < 1e-6)
    assert 0.0007 < frac < 0.0013
