"""Pins for the oracle's tensor-level flushes and dequantize.

The group rule is pinned in test_oracle_groups.py; here the fixtures pin the
gathering axis (keys group tokens of one channel, values group channels of
one token -- blog post "A 5.65x Metal Kernel That Made My LLM Exactly 0%
Faster", sections "What we're actually optimizing" and "The layout problem
that shapes everything"), the documented packed layout, token offsets, the
ragged key tail, and that dequantize reproduces the flush's reconstruction.
"""
import numpy as np
import pytest

from golden_io import hexes, rows

D = 128


def _expected_words(codes_sd: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes[S][D] by the documented layout: channel d of a token lives
    in word d // (32/bits) at bit offset bits * (d % (32/bits))."""
    per = 32 // bits
    S = codes_sd.shape[0]
    words = np.zeros((S, D // per), np.uint64)
    for d in range(D):
        words[:, d // per] |= codes_sd[:, d].astype(np.uint64) << np.uint64(bits * (d % per))
    return words.astype(np.uint32)


def _f16(a) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
def test_key_layout_fixture(orc, bits):
    L = (1 << bits) - 1
    s = np.arange(32)[:, None]
    d = np.arange(D)[None, :]
    codes = (s + d) % (L + 1)
    codes[0, :] = 0
    codes[1, :] = L           # every channel spans [0, L]: scale 1, zero 0
    x = _f16(codes)[None]
    st = orc.Store(orc.KEYS, 1, 32, D, bits)
    rec = orc.quantize_keys(x, st)
    assert np.all(st.scale == 1.0) and np.all(st.zero == 0.0)
    assert np.array_equal(st.codes[0], _expected_words(codes, bits))
    assert np.array_equal(rec, x)


@pytest.mark.parametrize("bits", [2, 4])
def test_value_layout_fixture(orc, bits):
    L = (1 << bits) - 1
    s = np.arange(40)[:, None]
    d = np.arange(D)[None, :]
    codes = (3 * s + d) % (L + 1)
    codes[:, 0::32] = 0
    codes[:, 1::32] = L       # every 32-channel group of every token spans [0, L]
    x = _f16(codes)[None]
    st = orc.Store(orc.VALUES, 1, 40, D, bits)
    rec = orc.quantize_values(x, st)
    assert st.scale.shape == (1, 40, 4)
    assert np.all(st.scale == 1.0) and np.all(st.zero == 0.0)
    assert np.array_equal(st.codes[0], _expected_words(codes, bits))
    assert np.array_equal(rec, x)


def test_axes_are_distinct(orc):
    """Channel d scaled by 2^(d%4) and token s by 2^(s%3): keys must take
    their range over the tokens of one channel, values over the channels of
    one group of one token."""
    s = np.arange(32)[:, None]
    d = np.arange(D)[None, :]
    base = ((s * 7 + d * 3) % 16).astype(np.float64)
    x = base * 2.0 ** (d % 4) * 2.0 ** (s % 3)
    xk = _f16(x)[None]
    assert np.array_equal(_w32(xk[0]), x)           # exact in fp16
    ks = orc.Store(orc.KEYS, 1, 32, D, 4)
    orc.quantize_keys(xk, ks)
    vs = orc.Store(orc.VALUES, 1, 32, D, 4)
    orc.quantize_values(xk, vs)
    f15 = np.float32(15)
    krange = (x.max(axis=0) - x.min(axis=0)).astype(np.float32)
    assert np.array_equal(ks.zero[0, 0], x.min(axis=0).astype(np.float32))
    assert np.array_equal(ks.scale[0, 0], krange / f15)
    xg = x.reshape(32, 4, 32)
    vrange = (xg.max(axis=2) - xg.min(axis=2)).astype(np.float32)
    assert np.array_equal(vs.zero[0], xg.min(axis=2).astype(np.float32))
    assert np.array_equal(vs.scale[0], vrange / f15)
    # the two axes give different metadata on this input
    assert not np.array_equal(ks.scale[0, 0][:4], vs.scale[0, :4, 0])


def _w32(u16):
    return u16.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("bits", [2, 4])
def test_tensor_flush_reduces_to_groups(orc, bits):
    """Each key group is the strided token slice of one channel and each value
    group the contiguous channel slice of one token."""
    rng = np.random.default_rng(5)
    BH, S = 3, 77
    x = _f16(rng.standard_normal((BH, S, D)) * np.where(rng.random(D) < 0.05, 10, 1))
    ks = orc.Store(orc.KEYS, BH, 96, D, bits)
    krec = orc.quantize_keys(x, ks)
    vs = orc.Store(orc.VALUES, BH, 96, D, bits)
    vrec = orc.quantize_values(x, vs)
    per = 32 // bits
    for _ in range(60):
        bh, dd, ss = int(rng.integers(BH)), int(rng.integers(D)), int(rng.integers(S))
        g = ss // 32
        sl = x[bh, g * 32:min(g * 32 + 32, S), dd]
        sc, ze, q, rec = orc.quantize_group(sl, bits)
        assert ks.scale[bh, g, dd] == sc and ks.zero[bh, g, dd] == ze
        i = ss - g * 32
        word = ks.codes[bh, ss, dd // per]
        assert (int(word) >> (bits * (dd % per))) & ((1 << bits) - 1) == q[i]
        assert krec[bh, ss, dd] == rec[i]
        j = dd // 32
        sl = x[bh, ss, j * 32:j * 32 + 32]
        sc, ze, q, rec = orc.quantize_group(sl, bits)
        assert vs.scale[bh, ss, j] == sc and vs.zero[bh, ss, j] == ze
        word = vs.codes[bh, ss, dd // per]
        assert (int(word) >> (bits * (dd % per))) & ((1 << bits) - 1) == q[dd - j * 32]
        assert vrec[bh, ss, dd] == rec[dd - j * 32]


def test_ragged_key_tail_fixture(orc):
    row = [r for r in rows("hand_groups.txt") if r[0] == "ragged_2bit"][0]
    xs = hexes(row[2])
    x = np.repeat(np.array(xs, np.uint16)[:, None], D, axis=1)[None]   # [1][3][D]
    st = orc.Store(orc.KEYS, 1, 32, D, 2)
    rec = orc.quantize_keys(x, st)
    assert np.all(st.zero[0, 0] == 1.0) and np.all(st.scale[0, 0] == 1.0)
    codes = np.repeat(np.array([0, 2, 3])[:, None], D, axis=1)
    assert np.array_equal(st.codes[0, :3], _expected_words(codes, 2))
    assert np.all(rec[0] == np.array(hexes(row[6]), np.uint16)[:, None])


@pytest.mark.parametrize("kind", ["keys", "values"])
def test_offset_window_only(orc, kind):
    rng = np.random.default_rng(11)
    BH, S, cap, off = 2, 64, 160, 64 if kind == "keys" else 37
    x = _f16(rng.standard_normal((BH, S, D)))
    K = orc.KEYS if kind == "keys" else orc.VALUES
    fn = orc.quantize_keys if kind == "keys" else orc.quantize_values
    st = orc.Store(K, BH, cap, D, 4, fill_codes=0xDEADBEEF, fill_meta=-7.0)
    rec = fn(x, st, off)
    fresh = orc.Store(K, BH, S, D, 4)
    rec0 = fn(x, fresh, 0)
    assert np.array_equal(rec, rec0)
    assert np.array_equal(st.codes[:, off:off + S], fresh.codes)
    assert np.all(st.codes[:, :off] == 0xDEADBEEF) and np.all(st.codes[:, off + S:] == 0xDEADBEEF)
    if kind == "keys":
        g0, g1 = off // 32, (off + S) // 32
    else:
        g0, g1 = off, off + S
    assert np.array_equal(st.scale[:, g0:g1], fresh.scale)
    assert np.array_equal(st.zero[:, g0:g1], fresh.zero)
    assert np.all(st.scale[:, :g0] == -7.0) and np.all(st.scale[:, g1:] == -7.0)


def test_key_offset_must_be_group_aligned(orc):
    x = np.zeros((1, 32, D), np.uint16)
    st = orc.Store(orc.KEYS, 1, 96, D, 4)
    with pytest.raises(ValueError):
        orc.quantize_keys(x, st, 16)


@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("bits", [2, 4])
def test_dequantize_reproduces_flush_recon(orc, kind, bits):
    rng = np.random.default_rng(21 + bits)
    BH, S = 2, 96
    x = _f16(rng.standard_normal((BH, S, D)) * 3)
    K = orc.KEYS if kind == "keys" else orc.VALUES
    fn = orc.quantize_keys if kind == "keys" else orc.quantize_values
    st = orc.Store(K, BH, S, D, bits)
    rec = fn(x, st)
    assert np.array_equal(orc.dequantize(st, 0, S), rec)
    assert np.array_equal(orc.dequantize(st, 40, 50), rec[:, 40:90])


def test_dequantize_hand_store(orc):
    """A store written by hand: codes 0..15 along the channels of token 0 and
    15..0 of token 1, one key group with scale 0.5 and zero -1 everywhere."""
    st = orc.Store(orc.KEYS, 1, 32, D, 4)
    c0 = np.arange(D) % 16
    c1 = 15 - c0
    st.codes[0, :2] = _expected_words(np.stack([c0, c1]), 4)
    st.scale[:] = 0.5
    st.zero[:] = -1.0
    out = orc.dequantize(st, 0, 2)
    want = _f16(np.stack([c0, c1]) * 0.5 - 1.0)
    assert np.array_equal(out[0], want)


def test_flush_count_matches_generation1_table(orc):
    """Blog post "A 5.65x Metal Kernel ...", "The full end-to-end record",
    Generation 1: prompts of 559, 2059 and 8209 tokens flush 512, 2016 and
    8160 tokens per layer with residual_length 32 and group size 32."""
    assert orc.flush_count(559, 32, 32) == 512
    assert orc.flush_count(2059, 32, 32) == 2016
    assert orc.flush_count(8209, 32, 32) == 8160
    assert orc.flush_count(32, 32, 32) == 0
    assert orc.flush_count(2048, 128, 32) == 1920
