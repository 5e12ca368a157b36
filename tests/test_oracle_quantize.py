"""Pins for oracle/quantize.py against what the mathematics fixes.

- nearest(): brute force over the table with exact rationals (Fraction), on
  random values, on every midpoint (ties go to the lower index) and on
  values one fp64 step either side of a midpoint;
- the uniform table with the ``range`` rule is asymmetric INT round-to-
  nearest: closed-form scale and ``clip(ceil(w/s - 1/2) + z, 0, L - 1)``;
- scales: all-zero groups, the fp16 clamp, an fp16 round-to-even tie, and
  the ``absmax`` rule landing the largest weight on the outermost entry;
- the weight error against a hand sum with exact rationals;
- the log table's values, and the base search recovering the base that
  generated the weights (error exactly 0) among other candidates;
- table tuning: one step against exact rational centroids, a table that is
  already the centroids of its own weights stays put, unused codes keep
  their entries, and the error of each table matches its own evaluation.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import quantize as Q


def _brute_nearest(r: float, T) -> int:
    rf = Fraction(r)
    d = [abs(rf - Fraction(float(t))) for t in T]
    best = min(d)
    return d.index(best)  # first (lowest) index among the minima


TABLES = {
    "nf4": np.array([-1.0, -0.6958, -0.5249, -0.3945, -0.2844, -0.1848, -0.0911, 0.0,
                     0.0796, 0.1609, 0.2461, 0.3379, 0.4407, 0.5626, 0.7229, 1.0], np.float16),
    "unsorted3": np.array([0.5, -1.5, 2.25, -0.25, 1.0, -3.0, 0.125, 3.5], np.float16),
    "int2": np.array([-2, -1, 0, 1], np.float16),
}


@pytest.mark.parametrize("name", list(TABLES))
def test_nearest_matches_exact_brute_force(name):
    T = TABLES[name]
    rng = np.random.default_rng(5)
    r = np.concatenate([rng.uniform(-4, 4, 400), rng.normal(0, 0.5, 200)])
    Ts = np.sort(T.astype(np.float64))
    mids = (Ts[:-1] + Ts[1:]) / 2
    r = np.concatenate([r, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        Ts, [-1e9, 1e9]])
    got = Q.nearest(r, T)
    want = [_brute_nearest(float(v), T) for v in r]
    assert list(got) == want


def test_nearest_ties_go_to_the_lower_index():
    T = np.array([1.0, 0.0, -1.0, 2.0], np.float16)   # 0.5 is between T[1]=0 and T[0]=1
    assert Q.nearest(np.array([0.5, -0.5, 1.5]), T).tolist() == [0, 1, 0]


def test_range_rule_on_uniform_table_is_int_rtn():
    rng = np.random.default_rng(6)
    for bits in (2, 3, 4):
        L, z = 1 << bits, 1 << (bits - 1)
        T = (np.arange(L) - z).astype(np.float16)
        w = (rng.normal(0, 0.02, (8, 256)) + rng.normal(0, 0.005, (8, 1))).astype(np.float32)
        c, s = Q.quantize(w, T, 128, "range")
        g = w.astype(np.float64).reshape(8, 2, 128)
        s_want = np.maximum(g.max(-1) / (L - 1 - z), -g.min(-1) / z).astype(np.float16)
        assert np.array_equal(s.view(np.uint16), s_want.view(np.uint16))
        r = g / s.astype(np.float64)[:, :, None]
        c_want = np.clip(np.ceil(r - 0.5) + z, 0, L - 1).astype(np.uint8).reshape(8, 256)
        assert np.array_equal(c, c_want)


def test_scale_edge_cases():
    T = np.array([-1.0, -0.5, 0.5, 1.0], np.float16)
    w = np.zeros((2, 256), np.float32)
    w[1, :128] = 1e6            # clamps to the largest finite fp16
    w[1, 128] = np.float32(1 + 2 ** -11)   # exactly halfway between two fp16 values
    s = Q.scales(w, T, 128, "absmax")
    assert s.dtype == np.float16 and s.shape == (2, 2)
    assert float(s[0, 0]) == 1.0 and float(s[0, 1]) == 1.0      # all-zero groups
    assert float(s[1, 0]) == 65504.0
    assert s[1, 1].view(np.uint16) == np.float16(1.0).view(np.uint16)   # tie -> even
    w[1, 129] = np.float32(1 + 3 * 2 ** -11)                            # tie -> even, upward
    assert float(Q.scales(w, T, 128, "absmax")[1, 1]) == float(np.float16(1 + 2 ** -9))
    with pytest.raises(ValueError):
        Q.scales(w, np.array([0.0, 1.0], np.float16), 128, "range")


def test_absmax_puts_the_largest_weight_on_the_outer_entry():
    rng = np.random.default_rng(7)
    T = TABLES["nf4"]
    w = rng.standard_t(4, (16, 512)).astype(np.float32)
    c, s = Q.quantize(w, T, 128, "absmax")
    g = np.abs(w).reshape(16, 4, 128)
    i = g.argmax(-1)
    for n in range(16):
        for j in range(4):
            k = j * 128 + i[n, j]
            assert c[n, k] == (15 if w[n, k] > 0 else 0)


def test_tensor_wise_equals_one_group():
    rng = np.random.default_rng(8)
    T = TABLES["unsorted3"]
    w = rng.normal(0, 1, (1, 384)).astype(np.float32)
    c0, s0 = Q.quantize(w, T, 0, "absmax")
    c1, s1 = Q.quantize(w, T, 384, "absmax")
    assert np.array_equal(c0, c1) and s0[0] == s1[0, 0]


def test_sq_error_matches_exact_sum():
    rng = np.random.default_rng(9)
    T = TABLES["unsorted3"]
    w = rng.normal(0, 1, (3, 256)).astype(np.float32)
    c, s = Q.quantize(w, T, 128, "absmax")
    want = Fraction(0)
    for n in range(3):
        for k in range(256):
            v = Fraction(float(T[c[n, k]])) * Fraction(float(s[n, k // 128]))
            want += (Fraction(float(w[n, k])) - v) ** 2
    assert abs(Q.sq_error(w, T, c, s, 128) - float(want)) <= 1e-12 * float(want)


def test_log_table_values():
    T = Q.log_table(4, 2.0)
    assert T.tolist() == [1, 0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125,
                          -1, -0.5, -0.25, -0.125, -0.0625, -0.03125, -0.015625, -0.0078125]
    T3 = Q.log_table(3, 1.5)
    assert np.allclose(T3.astype(np.float64), [1, 1 / 1.5, 1 / 2.25, 1 / 3.375,
                                                -1, -1 / 1.5, -1 / 2.25, -1 / 3.375], rtol=1e-3)


def test_log_base_search_recovers_the_generating_base():
    rng = np.random.default_rng(10)
    bases = [1.25, 2 ** 0.5, 1.6, 2.0]
    T = Q.log_table(4, 2 ** 0.5)
    c = rng.integers(0, 16, (32, 256))
    c[:, 0] = 0                                 # every group holds +1 * s: absmax = s
    w = (T[c].astype(np.float32) * np.float32(2 ** -5))
    best, errs = Q.log_base_search(w, 4, 128, bases)
    assert best == 1 and errs[1] == 0.0
    assert all(e > 0 for i, e in enumerate(errs) if i != 1)


def test_tune_one_step_is_the_exact_centroid():
    rng = np.random.default_rng(11)
    T0 = TABLES["nf4"]
    w = rng.normal(0, 0.3, (6, 256)).astype(np.float32)
    T1, s16, errs = Q.tune_table(w, T0, 128, "absmax", 1)
    c = Q.codes(w, T0, s16, 128)
    for i in range(16):
        num = den = Fraction(0)
        for n in range(6):
            for k in range(256):
                if c[n, k] == i:
                    sv = Fraction(float(s16[n, k // 128]))
                    num += Fraction(float(w[n, k])) * sv
                    den += sv * sv
        want = np.float16(float(num / den)) if den else T0[i]
        assert T1[i] == want, i
    assert len(errs) == 2


def test_tune_keeps_a_table_that_is_its_own_centroids():
    # every code's weights sit exactly on s * T[i], and each group holds +-s
    rng = np.random.default_rng(12)
    T0 = TABLES["nf4"]
    c = rng.integers(0, 16, (4, 256))
    c[:, 0] = 15
    c[:, 128] = 15
    s = (2.0 ** -rng.integers(3, 8, (4, 2))).astype(np.float32)
    w = (T0[c].astype(np.float32) * np.repeat(s, 128, axis=1)).astype(np.float32)
    T, _, errs = Q.tune_table(w, T0, 128, "absmax", 3)
    assert np.array_equal(T.view(np.uint16), T0.view(np.uint16))
    assert errs == [0.0] * 4


def test_tune_unused_codes_keep_their_entries_and_errors_are_consistent():
    rng = np.random.default_rng(13)
    T0 = TABLES["int2"]                       # -2 -1 0 1
    w = np.abs(rng.normal(0, 1, (3, 256))).astype(np.float32)    # never near -2 or -1
    T, s16, errs = Q.tune_table(w, T0, 0, "range", 4)
    assert T[0] == T0[0] and T[1] == T0[1]
    assert errs[-1] == Q.sq_error(w, T, Q.codes(w, T, s16, 0), s16, 0)
    assert errs[-1] <= errs[0]
