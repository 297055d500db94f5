"""Pins for the oracle's binary16-metadata store (scale and zero kept as
binary16; ORC_META_F16 in kivi_oracle.h).

Reading: the binary32 scale and zero of a group are rounded to nearest-even
binary16 for storage, and the codes and the reconstruction are taken with
the stored values (blog post "A 5.65x Metal Kernel That Made My LLM Exactly
0% Faster", "What we're actually optimizing", for the quantizer; the pages
leave the metadata precision open, and the VeloxQuant-MLX "Benchmarks"
page's KV-compression ratios depend on it).

What pins it, none of which is the oracle itself:
  * hand-worked groups (tests/golden/meta16_groups.txt), including a
    rounded scale that moves a code, a subnormal tie, a clip past the top
    code and a scale that underflows to 0;
  * an exact-rational emulation of every IEEE operation (tests/_exact.py)
    on random groups and at the tensor level, and a fixture row that the
    plausible wrong reading (codes from the binary32 scale) fails;
  * numpy's own binary16 rounding of the binary32-metadata store;
  * groups whose binary32 scale is a binary16 value reduce to the pinned
    binary32 path exactly;
  * invariants: code range, |x - recon| <= stored scale / 2 plus roundings,
    and dequantize reproducing the flush's reconstruction.
"""
import numpy as np
import pytest

import _exact as E
from golden_io import hexes, ints, rows

KEYS, VALUES = 0, 1


def _h16(v) -> int:
    return int(np.array([v], np.float32).astype(np.float16).view(np.uint16)[0])


@pytest.mark.parametrize("row", list(rows("meta16_groups.txt")), ids=lambda r: r[0])
def test_hand_worked_group(orc, row):
    name, bits, xs, scale, zero, codes, recon, codes32 = row
    bits = int(bits)
    x = np.array(hexes(xs), np.uint16)
    sc, ze, q, rec = orc.quantize_group(x, bits, meta="f16")
    # the widened values are binary16 values: the round trip is exact
    assert float(np.float32(sc).astype(np.float16)) == float(sc)
    assert _h16(sc) == int(scale, 16), name
    assert _h16(ze) == int(zero, 16), name
    assert list(q) == ints(codes), name
    assert list(rec) == hexes(recon), name
    # the same group with binary32 metadata
    _, _, q32, _ = orc.quantize_group(x, bits)
    assert list(q32) == ints(codes32), name


def test_fixture_separates_the_store_only_reading():
    """Rounding only for storage (codes from the binary32 scale) fails the
    first fixture row: its middle code is 7, not 8."""
    row = next(r for r in rows("meta16_groups.txt") if r[0] == "third_4bit")
    g = hexes(row[2])
    _, _, q, _ = E.quantize_group(g, 4, meta="f16_store_only")
    _, _, q16, _ = E.quantize_group(g, 4, meta="f16")
    assert q16 == ints(row[5]) and q != q16


@pytest.mark.parametrize("bits", [2, 4])
def test_random_groups_against_exact(orc, bits):
    rng = np.random.default_rng(410 + bits)
    for _ in range(250):
        n = int(rng.integers(1, 33))
        mag = 10.0 ** rng.uniform(-7, 4)          # reaches subnormal scales
        x = (rng.standard_normal(n) * mag).astype(np.float16).view(np.uint16)
        sc, ze, q, rec = orc.quantize_group(x, bits, meta="f16")
        esc, eze, eq, erec = E.quantize_group(list(x), bits, meta="f16")
        assert _h16(sc) == E.f16_bits(esc)
        assert _h16(ze) == E.f16_bits(eze)
        assert list(q) == eq
        assert list(rec) == erec


@pytest.mark.parametrize("bits", [2, 4])
def test_stored_pair_is_numpys_binary16_of_the_binary32_pair(orc, bits):
    rng = np.random.default_rng(5 + bits)
    x = (rng.standard_normal((6, 64, 128)) * 3).astype(np.float16)
    for kind, quant in ((KEYS, orc.quantize_keys), (VALUES, orc.quantize_values)):
        s32 = orc.Store(kind, 6, 64, bits=bits)
        s16 = orc.Store(kind, 6, 64, bits=bits, meta="f16")
        quant(x, s32)
        quant(x, s16)
        assert np.array_equal(s16.scale, s32.scale.astype(np.float16).astype(np.float32))
        assert np.array_equal(s16.zero, s32.zero)          # an fp16 minimum is exact
        sb, zb = s16.meta_bits()
        assert np.array_equal(sb, s32.scale.astype(np.float16).view(np.uint16))
        # the rounded scale moves some codes, so the variant is not a no-op
        assert not np.array_equal(s16.codes, s32.codes)


@pytest.mark.parametrize("bits", [2, 4])
def test_binary16_exact_scales_reduce_to_the_binary32_path(orc, bits):
    """Integer-valued groups whose range is L * 2^k: the binary32 scale 2^k is
    a binary16 value, so both stores hold identical codes, scales, zeros and
    reconstructions."""
    rng = np.random.default_rng(77 + bits)
    L = (1 << bits) - 1
    x = np.zeros((4, 64, 128), np.float32)
    for bh in range(4):
        for g in range(2):
            k = 2.0 ** int(rng.integers(-3, 3))
            c = float(rng.integers(-20, 20)) * k
            lv = rng.integers(0, L + 1, size=(32, 128)).astype(np.float32)
            lv[0, :], lv[1, :] = 0, L                        # every channel's range is L * k
            x[bh, 32 * g:32 * g + 32] = c + lv * k
    x16 = x.astype(np.float16)
    s32 = orc.Store(KEYS, 4, 64, bits=bits)
    s16 = orc.Store(KEYS, 4, 64, bits=bits, meta="f16")
    r32 = orc.quantize_keys(x16, s32)
    r16 = orc.quantize_keys(x16, s16)
    assert np.array_equal(s32.scale, s16.scale) and np.array_equal(s32.codes, s16.codes)
    assert np.array_equal(r32, r16)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", [KEYS, VALUES])
def test_tensor_flush_against_exact_and_invariants(orc, bits, kind):
    rng = np.random.default_rng(900 + 2 * bits + kind)
    BH, S, D, G = 2, 40, 128, 32                        # a ragged last key group
    x = (rng.standard_normal((BH, S, D)) * rng.uniform(1e-3, 4)).astype(np.float16)
    st = orc.Store(kind, BH, 64, bits=bits, meta="f16")
    quant = orc.quantize_keys if kind == KEYS else orc.quantize_values
    rec = quant(x, st)
    L = (1 << bits) - 1
    xb = x.view(np.uint16)
    # exact emulation of a sample of groups
    for bh in range(BH):
        for gi in range(6):
            if kind == KEYS:
                g0, d = 32 * int(rng.integers(0, 2)), int(rng.integers(0, D))
                grp = list(xb[bh, g0:min(g0 + G, S), d])
                sc, ze = st.scale[bh, g0 // G, d], st.zero[bh, g0 // G, d]
                w = d * bits // 32
                sh = (d % (32 // bits)) * bits
                q = [(int(st.codes[bh, t, w]) >> sh) & L for t in range(g0, g0 + len(grp))]
                r = list(rec[bh, g0:g0 + len(grp), d])
            else:
                t, j = int(rng.integers(0, S)), int(rng.integers(0, D // G))
                grp = list(xb[bh, t, G * j:G * j + G])
                sc, ze = st.scale[bh, t, j], st.zero[bh, t, j]
                q = []
                for d in range(G * j, G * j + G):
                    w, sh = d * bits // 32, (d % (32 // bits)) * bits
                    q.append((int(st.codes[bh, t, w]) >> sh) & L)
                r = list(rec[bh, t, G * j:G * j + G])
            esc, eze, eq, erec = E.quantize_group(grp, bits, meta="f16")
            assert _h16(sc) == E.f16_bits(esc) and _h16(ze) == E.f16_bits(eze)
            assert q == eq and [int(v) for v in r] == erec
    # |x - recon| <= s/2 + roundings for normal binary16 scales: the rounded
    # scale is within 2^-11 of range/L, so the top level L*s misses the
    # maximum by at most L * s * 2^-11 < s/2
    xs = x.astype(np.float64)
    rs = rec.view(np.float16).astype(np.float64)
    if kind == KEYS:
        s_el = np.repeat(st.scale[:, :2, :], G, axis=1)[:, :S, :].astype(np.float64)
    else:
        s_el = np.repeat(st.scale[:, :S, :], G, axis=2).astype(np.float64)
    ok = s_el >= 2.0 ** -14
    ulp = np.spacing(np.abs(rs).astype(np.float16)).astype(np.float64)
    slack = 0.5 * ulp + 2.0 ** -21 * (np.abs(xs) + L * s_el)
    assert np.all((np.abs(xs - rs) <= s_el / 2 + slack)[ok])
    # dequantize reads the stored pair and reproduces the flush's reconstruction
    assert np.array_equal(orc.dequantize(st, 0, S), rec)


def test_bf16_inputs_are_refused(orc):
    st = orc.Store(KEYS, 1, 32, meta="f16")
    with pytest.raises(ValueError):
        orc.quantize_keys(np.zeros((1, 32, 128), np.uint16), st, fmt="bf16")


def test_attend_over_a_binary16_store_matches_dense_attention(orc):
    """The attend reads the stored (widened) pair, so it equals softmax(qK^T)V
    over dequantize's reconstruction, evaluated here with numpy in float64."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, D, nq, nr = 2, 8, 2, 128, 64, 5
    k = (rng.standard_normal((B * Hkv, nq, D))).astype(np.float16)
    v = (rng.standard_normal((B * Hkv, nq, D))).astype(np.float16)
    ks = orc.Store(KEYS, B * Hkv, nq, meta="f16")
    vs = orc.Store(VALUES, B * Hkv, nq, meta="f16")
    orc.quantize_keys(k, ks)
    orc.quantize_values(v, vs)
    kr = (rng.standard_normal((B * Hkv, 8, D))).astype(np.float16)
    vr = (rng.standard_normal((B * Hkv, 8, D))).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    out = orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr)
    K = np.concatenate([orc.dequantize(ks, 0, nq).view(np.float16), kr[:, :nr]], axis=1)
    V = np.concatenate([orc.dequantize(vs, 0, nq).view(np.float16), vr[:, :nr]], axis=1)
    K, V = K.astype(np.float64), V.astype(np.float64)
    qq = q.astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            kv = b * Hkv + h // (Hq // Hkv)
            s = K[kv] @ qq[b, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ V[kv]
            assert np.allclose(out[b, h], want, rtol=1e-12, atol=1e-12)
