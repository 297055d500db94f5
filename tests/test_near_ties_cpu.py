"""The near-tie generator (tests/near_ties.py) and the oracle at near ties.

The generator is checked with the exact-rational emulation (tests/_exact.py,
which shares no arithmetic with numpy or the oracle): every group holds its
min and max, and its other 30 elements have a binary32 quotient within
2^-12 of a half-integer.  On the same groups the oracle must equal the
emulation bit for bit -- the quantizer's steps at exactly the inputs where
rounding decides the code ([Metal post] "Three ways to be off by one bit")."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import _exact
from near_ties import NEAR, as_keys, as_values, near_tie_groups

CASES = [(4, "f16", "f32"), (2, "f16", "f32"), (4, "f16", "f16"), (2, "f16", "f16"),
         (4, "bf16", "f32"), (2, "bf16", "f32")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d-%s-meta%s" % c)
def test_groups_are_near_ties_and_oracle_matches_exact(case):
    bits, fmt, meta = case
    groups, n_near = near_tie_groups(120, bits, seed=5, fmt=fmt, meta=meta)
    assert groups.shape == (120, 32) and n_near == 120 * 30
    value = _exact.f16_value if fmt == "f16" else _exact.bf16_value
    levels = (1 << bits) - 1
    exact_ties = 0
    for g in groups:
        xs = [value(b) for b in g]
        mn, mx = min(xs), max(xs)
        scale = _exact.rnd32(_exact.rnd32(mx - mn) / levels)
        if meta == "f16":
            scale = _exact.rnd16(scale)
        near = 0
        for x in xs:
            if x in (mn, mx):
                continue
            u = _exact.rnd32(_exact.rnd32(x - mn) / scale)
            d = abs(u - (u.numerator // u.denominator) - Fraction(1, 2))
            assert d <= Fraction(NEAR), (g, x, float(u))
            exact_ties += d == 0
            near += 1
        assert near >= 30 - sum(x in (mn, mx) for x in xs[2:])   # duplicates of min/max aside
        sc, ze, q, rec = oracle.quantize_group(g, bits, fmt=fmt, meta=meta)
        esc, eze, eq, erec = _exact.quantize_group(g, bits, fmt=fmt, meta=meta)
        assert Fraction(float(sc)) == esc and Fraction(float(ze)) == eze
        assert list(q) == eq, g
        assert list(rec) == erec, g
    assert exact_ties > 0            # exact half-integer quotients occur too


def test_layouts_put_each_group_in_place():
    groups = np.arange(2 * 64 * 128 // 32 * 32, dtype=np.uint16).reshape(-1, 32)
    k = as_keys(groups, 2, 64, 128)
    assert np.array_equal(k[1, 32:64, 5], groups[(1 * 2 + 1) * 128 + 5])
    v = as_values(groups, 2, 64, 128)
    assert np.array_equal(v[1, 7, 64:96], groups[(1 * 64 + 7) * 4 + 2])
