"""Pins for the oracle's one-group quantizer (orc_quantize_group).

What pins it, none of which is the oracle itself:
  * hand-worked groups (tests/golden/hand_groups.txt), derived by hand from
    the rule in the blog post "A 5.65x Metal Kernel That Made My LLM Exactly
    0% Faster" ("What we're actually optimizing"; "Three ways to be off by
    one bit");
  * groups that separate the chosen reading from a plausible wrong one
    (tests/golden/regression_triples.txt), checked against an exact-rational
    emulation of every IEEE operation (tests/_exact.py);
  * brute force over every small group drawn from an alphabet of awkward
    fp16 values, against the same emulation;
  * invariants of the rule: code range, exact reconstruction of the group
    minimum, the error bound, order independence, monotonicity and exact
    scaling by powers of two.
"""
import itertools

import numpy as np
import pytest

import _exact as E
from golden_io import hexes, ints, rows


def _f32_bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


@pytest.mark.parametrize("row", list(rows("hand_groups.txt")), ids=lambda r: r[0])
def test_hand_worked_group(orc, row):
    name, bits, xs, scale, zero, codes, recon = row
    bits = int(bits)
    sc, ze, q, rec = orc.quantize_group(np.array(hexes(xs), np.uint16), bits)
    assert _f32_bits(sc) == int(scale, 16), name
    assert _f32_bits(ze) == int(zero, 16), name
    assert list(q) == ints(codes), name
    assert list(rec) == hexes(recon), name


@pytest.mark.parametrize("row", list(rows("regression_triples.txt")),
                         ids=lambda r: "-".join(r))
def test_regression_triple(orc, row):
    bits, mn, mx, x, wrong = row
    bits = int(bits)
    g = [int(mn, 16), int(mx, 16), int(x, 16)]
    sc, ze, q, rec = orc.quantize_group(np.array(g, np.uint16), bits)
    esc, eze, eq, erec = E.quantize_group(g, bits)
    assert _f32_bits(sc) == E.f32_bits(esc)
    assert _f32_bits(ze) == E.f32_bits(eze)
    assert list(q) == eq
    assert list(rec) == erec
    kw = {"away": dict(ties="away"), "exact": dict(quotient="exact"),
          "rcp": dict(quotient="rcp"), "fma": dict(recon_fma=True)}[wrong]
    _, _, wq, wrec = E.quantize_group(g, bits, **kw)
    if wrong == "fma":
        assert wrec[2] != erec[2], "fixture does not separate the FMA reading"
    else:
        assert wq[2] != eq[2], "fixture does not separate the %s reading" % wrong


# fp16 alphabet: signed zeros, subnormals, the largest finite values,
# dyadic ties, non-dyadic fractions and a few N(0,1)-like values.
_ALPHABET = [0x0000, 0x8000, 0x0001, 0x03FF, 0x8200, 0x7BFF, 0xFBFF,
             0x3800, 0x3E00, 0x4100, 0xB800, 0x3C00, 0xBC00, 0x2E66,
             0x34CD, 0x3ECD, 0xBE50, 0x3EA6, 0xBC27, 0xC09F, 0x414A,
             0x30E0, 0x4B80, 0x5640]


def _check_against_exact(orc, g, bits):
    sc, ze, q, rec = orc.quantize_group(np.array(g, np.uint16), bits)
    esc, eze, eq, erec = E.quantize_group(g, bits)
    assert _f32_bits(sc) == E.f32_bits(esc), g
    assert _f32_bits(ze) == E.f32_bits(eze) or (ze == 0 and eze == 0), g
    assert list(q) == eq, g
    assert list(rec) == erec, g


@pytest.mark.parametrize("bits", [2, 4])
def test_brute_force_pairs_and_triples(orc, bits):
    alpha = _ALPHABET
    for n in (1, 2):
        for g in itertools.product(alpha, repeat=n):
            _check_against_exact(orc, list(g), bits)
    sub = alpha[::2]
    for g in itertools.product(sub, repeat=3):
        _check_against_exact(orc, list(g), bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_random_groups_against_exact(orc, bits):
    rng = np.random.default_rng(99 + bits)
    for _ in range(300):
        n = int(rng.integers(1, 33))
        scale = 10.0 ** rng.uniform(-3, 3)
        x = (rng.standard_normal(n) * scale).astype(np.float16)
        _check_against_exact(orc, list(x.view(np.uint16)), bits)


def _random_groups(rng, count, n, outliers=False):
    x = rng.standard_normal((count, n)).astype(np.float32)
    if outliers:
        x[: count // 4] *= 10.0
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
def test_invariants(orc, bits):
    rng = np.random.default_rng(7 + bits)
    L = (1 << bits) - 1
    groups = _random_groups(rng, 3000, 32, outliers=True)
    for g in groups:
        sc, ze, q, rec = orc.quantize_group(g, bits)
        x = orc.f16_to_f32(g).astype(np.float64)
        r = orc.f16_to_f32(rec).astype(np.float64)
        assert q.min() >= 0 and q.max() <= L
        # the minimum is the zero point and is reconstructed exactly; the
        # maximum gets the top code
        assert float(ze) == x.min()
        assert np.all(q[x == x.min()] == 0) and np.all(rec[x == x.min()] == g[x == x.min()])
        assert np.all(q[x == x.max()] == L)
        # |x - recon| <= scale/2, up to the fp32 rounding of the operations
        # and the fp16 rounding of the output
        ulp16 = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
        slack = 0.5 * ulp16 + 2.0 ** -22 * (abs(float(ze)) + L * float(sc))
        assert np.all(np.abs(x - r) <= float(sc) / 2 + slack)
        # monotone: a larger input never gets a smaller code
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order].astype(int)) >= 0)
        # order independence
        perm = rng.permutation(32)
        sc2, ze2, q2, rec2 = orc.quantize_group(g[perm], bits)
        assert sc2 == sc and ze2 == ze
        assert np.array_equal(q2, q[perm]) and np.array_equal(rec2, rec[perm])


@pytest.mark.parametrize("bits", [2, 4])
def test_power_of_two_scaling(orc, bits):
    """Scaling a group by 2^k is exact in every step (no overflow or
    underflow), so codes are unchanged and scale, zero and recon scale by 2^k."""
    rng = np.random.default_rng(3)
    groups = _random_groups(rng, 500, 32)
    checked = 0
    for g in groups:
        x = g.view(np.float16).astype(np.float32)
        for k in (-3, 4):
            y = (x * np.float32(2.0 ** k)).astype(np.float16)
            if not np.array_equal(y.astype(np.float32), x * np.float32(2.0 ** k)):
                continue  # an input fell into the fp16 subnormal range
            checked += 1
            sc, ze, q, rec = orc.quantize_group(g, bits)
            sc2, ze2, q2, rec2 = orc.quantize_group(y.view(np.uint16), bits)
            assert np.array_equal(q2, q)
            assert sc2 == np.float32(sc * np.float32(2.0 ** k))
            assert ze2 == np.float32(ze * np.float32(2.0 ** k))
            # recon scales exactly unless either side lands in the fp16
            # subnormal range, where the rounding quantum stops scaling
            r0 = rec.view(np.float16).astype(np.float32)
            r1 = r0 * np.float32(2.0 ** k)
            r2 = rec2.view(np.float16).astype(np.float32)
            normal = np.minimum(np.abs(r0), np.abs(r1)) >= 2.0 ** -14
            assert np.array_equal(r2[normal], r1[normal])
    assert checked > 300


def test_constant_and_signed_zero_groups(orc):
    for bits in (2, 4):
        sc, ze, q, rec = orc.quantize_group(np.array([0x8000, 0x0000, 0x8000], np.uint16), bits)
        assert sc == 0 and _f32_bits(ze) == 0 and list(q) == [0, 0, 0]
        # a zero extreme is stored as +0 whichever zero came first
        sc, ze, q, rec = orc.quantize_group(np.array([0x8000, 0x3C00], np.uint16), bits)
        assert _f32_bits(ze) == 0 and list(q) == [0, (1 << bits) - 1]


def test_dequantize_one_matches_hand_values(orc):
    # q*scale is rounded before +zero: 7 * RN32(1/15) = 0.46666669 -> 0x3777
    assert orc.dequantize_one(7, np.uint32(0x3D888889).view(np.float32), 0.0) == 0x3777
    # 3 * 1.0 + (-2.0) = 1.0
    assert orc.dequantize_one(3, 1.0, -2.0) == 0x3C00
    # code 0 returns the zero point itself (rounded to fp16)
    assert orc.dequantize_one(0, 5.0, np.float32(0.7001953125)) == 0x399A
