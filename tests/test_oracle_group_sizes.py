"""Pins for the oracle's flushes with groups of 64 and 128 (the pages' cache
takes `group_size` as a parameter; the benchmark workloads use 32).

Each tensor-level group reduces to the group function on exactly its
elements: keys over G consecutive tokens of one channel (a ragged last group
over its real tokens), values over G consecutive channels of one token.  The
group function itself is pinned in test_oracle_groups.py."""
import numpy as np
import pytest

D = 128


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("bits", [2, 4])
def test_wide_groups_reduce_to_the_group_function(orc, G, bits):
    rng = np.random.default_rng(G + bits)
    BH, S = 2, 2 * G + 37                          # two whole key groups and a ragged one
    x = _f16(rng.standard_normal((BH, S, D)) * np.where(rng.random(D) < 0.05, 10, 1))
    cap = 3 * G
    ks = orc.Store(orc.KEYS, BH, cap, D, bits, G)
    vs = orc.Store(orc.VALUES, BH, cap, D, bits, G)
    rk = orc.quantize_keys(x, ks, 0)
    rv = orc.quantize_values(x, vs, 0)
    assert ks.scale.shape == (BH, 3, D) and vs.scale.shape == (BH, cap, D // G)
    for bh in range(BH):
        for g in range(3):
            s0, s1 = G * g, min(G * g + G, S)
            for d in (0, 63, 127):
                sc, ze, q, rec = orc.quantize_group(x[bh, s0:s1, d], bits)
                assert ks.scale[bh, g, d] == sc and ks.zero[bh, g, d] == ze
                assert np.array_equal(rk[bh, s0:s1, d], rec)
        for s in (0, G, S - 1):
            for j in range(D // G):
                sc, ze, q, rec = orc.quantize_group(x[bh, s, G * j:G * j + G], bits)
                assert vs.scale[bh, s, j] == sc and vs.zero[bh, s, j] == ze
                assert np.array_equal(rv[bh, s, G * j:G * j + G], rec)
    assert np.array_equal(orc.dequantize(ks, 0, S), rk)
    assert np.array_equal(orc.dequantize(vs, 0, S), rv)


def test_group_of_128_values_is_the_whole_row(orc):
    """With G = D every token has one value group: its scale is the row's
    (max - min) / (2^bits - 1)."""
    rng = np.random.default_rng(5)
    x = _f16(rng.standard_normal((1, 3, D)))
    vs = orc.Store(orc.VALUES, 1, 32, D, 4, 128)
    orc.quantize_values(x, vs, 0)
    w = x.view(np.float16).astype(np.float32)
    for s in range(3):
        assert vs.zero[0, s, 0] == w[0, s].min()
        assert vs.scale[0, s, 0] == np.float32(np.float32(w[0, s].max() - w[0, s].min()) / np.float32(15))


@pytest.mark.parametrize("G", [64, 128])
def test_attend_over_wide_group_stores_matches_torch_sdpa(orc, G):
    """The attend over stores with groups of G is the definition over their
    dequantized tokens (torch float64 SDPA, a library routine)."""
    import torch
    rng = np.random.default_rng(G)
    B, Hq, Hkv, nq, nr = 2, 8, 2, 150, 11
    cap = ((nq + G - 1) // G) * G
    k = _f16(rng.standard_normal((B * Hkv, nq, D)) * np.where(rng.random(D) < 0.05, 10, 1))
    v = _f16(rng.standard_normal((B * Hkv, nq, D)))
    ks = orc.Store(orc.KEYS, B * Hkv, cap, D, 4, G)
    vs = orc.Store(orc.VALUES, B * Hkv, cap, D, 4, G)
    orc.quantize_keys(k, ks)
    orc.quantize_values(v, vs)
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, 16, D)))
    vr = _f16(rng.standard_normal((B * Hkv, 16, D)))
    got = orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr)

    def w(u):
        return u.view(np.float16).astype(np.float64)
    kk = np.concatenate([w(orc.dequantize(ks, 0, nq)), w(kr[:, :nr])], axis=1)
    vv = np.concatenate([w(orc.dequantize(vs, 0, nq)), w(vr[:, :nr])], axis=1)
    g = Hq // Hkv
    kt = torch.from_numpy(kk.reshape(B, Hkv, -1, D)).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(vv.reshape(B, Hkv, -1, D)).repeat_interleave(g, dim=1)
    qt = torch.from_numpy(w(q)).reshape(B, Hq, 1, D)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(B, Hq, D).numpy()
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("Dh", [64, 256])
@pytest.mark.parametrize("bits", [2, 4])
def test_other_head_dims_reduce_to_the_group_function(orc, Dh, bits):
    """head_dim 64 and 256 with groups of 32: keys over 32 tokens of one of
    the Dh channels, values over 32 channels of a token (Dh/32 groups)."""
    rng = np.random.default_rng(Dh + bits)
    BH, S, G = 2, 70, 32
    x = _f16(rng.standard_normal((BH, S, Dh)) * np.where(rng.random(Dh) < 0.05, 10, 1))
    ks = orc.Store(orc.KEYS, BH, 96, Dh, bits, G)
    vs = orc.Store(orc.VALUES, BH, 96, Dh, bits, G)
    rk = orc.quantize_keys(x, ks, 0)
    rv = orc.quantize_values(x, vs, 0)
    assert ks.codes.shape == (BH, 96, Dh * bits // 32) and vs.scale.shape == (BH, 96, Dh // G)
    for bh in range(BH):
        for g in range(3):
            s0, s1 = G * g, min(G * g + G, S)
            for d in (0, Dh // 2 + 1, Dh - 1):
                sc, ze, q, rec = orc.quantize_group(x[bh, s0:s1, d], bits)
                assert ks.scale[bh, g, d] == sc and ks.zero[bh, g, d] == ze
                assert np.array_equal(rk[bh, s0:s1, d], rec)
        for s in (0, 33, S - 1):
            for j in range(Dh // G):
                sc, ze, q, rec = orc.quantize_group(x[bh, s, G * j:G * j + G], bits)
                assert vs.scale[bh, s, j] == sc and vs.zero[bh, s, j] == ze
                assert np.array_equal(rv[bh, s, G * j:G * j + G], rec)
    assert np.array_equal(orc.dequantize(ks, 0, S), rk)
    assert np.array_equal(orc.dequantize(vs, 0, S), rv)


@pytest.mark.parametrize("D", [48, 80, 96, 112])
@pytest.mark.parametrize("bits", [2, 4])
def test_ragged_head_dims_reduce_to_the_group_function(orc, D, bits):
    """head_dims that 32 does not divide (or that are not 64, 128 or 256):
    every value group, the last one of 16 channels included, and every key
    group is the one-group quantizer on exactly its elements ([Metal post]
    "Kernel B": a token's group j is channels [32j, min(32j + 32, D)))."""
    rng = np.random.default_rng(D + bits)
    BH, S, G = 2, 45, 32
    x = (rng.standard_normal((BH, S, D)) * 2).astype(np.float16)
    xb = x.view(np.uint16)
    L = (1 << bits) - 1
    vs = orc.Store(orc.VALUES, BH, 64, D, bits, G)
    vrec = orc.quantize_values(xb, vs)
    assert vs.scale.shape == (BH, 64, (D + G - 1) // G)
    for bh in range(BH):
        for t in (0, 17, 44):
            for j in range((D + G - 1) // G):
                d0, d1 = G * j, min(G * j + G, D)
                sc, ze, q, rec = orc.quantize_group(xb[bh, t, d0:d1], bits)
                assert vs.scale[bh, t, j] == sc and vs.zero[bh, t, j] == ze
                got = [(int(vs.codes[bh, t, d * bits // 32]) >> ((d % (32 // bits)) * bits)) & L
                       for d in range(d0, d1)]
                assert got == list(q)
                assert np.array_equal(vrec[bh, t, d0:d1], rec)
    ks = orc.Store(orc.KEYS, BH, 64, D, bits, G)
    krec = orc.quantize_keys(xb, ks)
    for bh in range(BH):
        for g in range(2):
            t1 = min(G * g + G, S)
            for d in (0, D // 2, D - 1):
                sc, ze, q, rec = orc.quantize_group(xb[bh, G * g:t1, d], bits)
                assert ks.scale[bh, g, d] == sc and ks.zero[bh, g, d] == ze
                assert np.array_equal(krec[bh, G * g:t1, d], rec)
    assert np.array_equal(orc.dequantize(vs, 0, S), vrec)
    assert np.array_equal(orc.dequantize(ks, 0, S), krec)
