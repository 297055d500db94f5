"""Pins for the oracle's dequantize-then-attend (orc_decode_attend).

The oracle evaluates the definition softmax(q K^T / sqrt(D)) V in double
over the fp16 reconstruction of the store followed by the fp16 residual
window.  It is pinned by:
  * torch's float64 scaled_dot_product_attention (a library routine) on the
    residual-only case, with grouped-query heads expanded explicitly;
  * the same library routine over the oracle's dequantized store (which is
    pinned on its own in test_oracle_tensor.py);
  * closed forms: a single token returns its value row, a zero query returns
    the mean of all value rows, and a common shift of every key leaves the
    output unchanged.
"""
import numpy as np
import pytest
import torch

D = 128


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def _w(u16):
    return u16.view(np.float16).astype(np.float64)


def _sdpa(q, k, v, group):
    """q [B][Hq][D], k/v [B*Hkv][N][D] (float64) -> [B][Hq][D]."""
    B, Hq, _ = q.shape
    Hkv = Hq // group
    N = k.shape[1]
    kt = torch.from_numpy(k.reshape(B, Hkv, N, D)).repeat_interleave(group, dim=1)
    vt = torch.from_numpy(v.reshape(B, Hkv, N, D)).repeat_interleave(group, dim=1)
    qt = torch.from_numpy(q).reshape(B, Hq, 1, D)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.reshape(B, Hq, D).numpy()


def _stores(orc, rng, BH, n_quant, bits=4):
    k = _f16(rng.standard_normal((BH, n_quant, D)) * np.where(rng.random(D) < 0.04, 10, 1))
    v = _f16(rng.standard_normal((BH, n_quant, D)))
    ks = orc.Store(orc.KEYS, BH, ((n_quant + 31) // 32) * 32, D, bits)
    vs = orc.Store(orc.VALUES, BH, ks.cap, D, bits)
    orc.quantize_keys(k, ks)
    orc.quantize_values(v, vs)
    return ks, vs


@pytest.mark.parametrize("B,Hq,Hkv", [(1, 4, 1), (2, 8, 2), (1, 32, 8)])
def test_residual_only_matches_torch_sdpa(orc, B, Hq, Hkv):
    rng = np.random.default_rng(B * 100 + Hq)
    N = 37
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, N, D)))
    vr = _f16(rng.standard_normal((B * Hkv, N, D)))
    got = orc.decode_attend(q, B, Hq, Hkv, None, None, 0, kr, vr, N)
    want = _sdpa(_w(q), _w(kr), _w(vr), Hq // Hkv)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("bits", [2, 4])
def test_store_plus_residual_matches_torch_sdpa(orc, bits):
    rng = np.random.default_rng(40 + bits)
    B, Hq, Hkv, nq, nr = 2, 8, 2, 70, 20
    ks, vs = _stores(orc, rng, B * Hkv, nq, bits)
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, 32, D)))
    vr = _f16(rng.standard_normal((B * Hkv, 32, D)))
    got = orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr)
    kk = np.concatenate([_w(orc.dequantize(ks, 0, nq)), _w(kr[:, :nr])], axis=1)
    vv = np.concatenate([_w(orc.dequantize(vs, 0, nq)), _w(vr[:, :nr])], axis=1)
    want = _sdpa(_w(q), kk, vv, Hq // Hkv)
    assert np.max(np.abs(got - want)) < 1e-12


def test_single_token_returns_its_value(orc):
    rng = np.random.default_rng(1)
    q = _f16(rng.standard_normal((1, 4, D)) * 5)
    kr = _f16(rng.standard_normal((1, 1, D)))
    vr = _f16(rng.standard_normal((1, 1, D)))
    got = orc.decode_attend(q, 1, 4, 1, None, None, 0, kr, vr, 1)
    assert np.array_equal(got, np.broadcast_to(_w(vr[0]), (1, 4, D)))
    ks, vs = _stores(orc, rng, 1, 1)
    got = orc.decode_attend(q, 1, 4, 1, ks, vs, 1, None, None, 0)
    assert np.array_equal(got, np.broadcast_to(_w(orc.dequantize(vs, 0, 1)[0]), (1, 4, D)))


def test_zero_query_gives_mean_of_values(orc):
    rng = np.random.default_rng(2)
    nq, nr = 64, 9
    ks, vs = _stores(orc, rng, 1, nq)
    q = np.zeros((1, 4, D), np.uint16)
    kr = _f16(rng.standard_normal((1, 16, D)))
    vr = _f16(rng.standard_normal((1, 16, D)))
    got = orc.decode_attend(q, 1, 4, 1, ks, vs, nq, kr, vr, nr)
    vv = np.concatenate([_w(orc.dequantize(vs, 0, nq)[0]), _w(vr[0, :nr])], axis=0)
    assert np.max(np.abs(got[0] - vv.mean(axis=0))) < 1e-13


def test_common_key_shift_leaves_output_unchanged(orc):
    """Adding one vector a to every key adds q.a to every score."""
    rng = np.random.default_rng(3)
    N = 50
    k = rng.integers(-4, 5, size=(1, N, D)).astype(np.float32)
    a = rng.integers(-8, 9, size=(1, 1, D)).astype(np.float32)
    q = _f16(rng.standard_normal((1, 4, D)) * 0.3)
    v = _f16(rng.standard_normal((1, N, D)))
    o1 = orc.decode_attend(q, 1, 4, 1, None, None, 0, _f16(k), v, N)
    o2 = orc.decode_attend(q, 1, 4, 1, None, None, 0, _f16(k + a), v, N)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_varlen_matches_torch_sdpa_per_sequence(orc):
    """Each sequence attends over its own prefix of the store and of the
    residual window: torch's float64 SDPA on exactly those rows."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, cap, R = 4, 8, 2, 96, 24
    ks, vs = _stores(orc, rng, B * Hkv, cap)
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, R, D)))
    vr = _f16(rng.standard_normal((B * Hkv, R, D)))
    nq = np.array([96, 0, 33, 70], np.int32)
    nr = np.array([0, 24, 7, 24], np.int32)
    got = orc.decode_attend_varlen(q, B, Hq, Hkv, ks, vs, nq, cap, kr, vr, nr, R)
    kd, vd = _w(orc.dequantize(ks, 0, cap)), _w(orc.dequantize(vs, 0, cap))
    for b in range(B):
        sl = slice(b * Hkv, (b + 1) * Hkv)
        kk = np.concatenate([kd[sl, :nq[b]], _w(kr[sl, :nr[b]])], axis=1)
        vv = np.concatenate([vd[sl, :nq[b]], _w(vr[sl, :nr[b]])], axis=1)
        want = _sdpa(_w(q[b:b + 1]), kk, vv, Hq // Hkv)[0]
        assert np.max(np.abs(got[b] - want)) < 1e-12, b


def test_varlen_equal_lengths_is_the_uniform_call(orc):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, nq, nr = 3, 8, 2, 64, 9
    ks, vs = _stores(orc, rng, B * Hkv, nq)
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, 16, D)))
    vr = _f16(rng.standard_normal((B * Hkv, 16, D)))
    want = orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr)
    got = orc.decode_attend_varlen(q, B, Hq, Hkv, ks, vs, np.full(B, nq), nq, kr, vr,
                                   np.full(B, nr), 16)
    assert np.array_equal(got, want)


def test_varlen_clamps_lengths_and_zeroes_empty_sequences(orc):
    """Lengths are clamped to [0, max]; a sequence left empty outputs 0."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, cap = 3, 4, 1, 64
    ks, vs = _stores(orc, rng, B * Hkv, cap)
    q = _f16(rng.standard_normal((B, Hq, D)))
    kr = _f16(rng.standard_normal((B * Hkv, 8, D)))
    vr = _f16(rng.standard_normal((B * Hkv, 8, D)))
    got = orc.decode_attend_varlen(q, B, Hq, Hkv, ks, vs, np.array([1000, -5, 0]), 40, kr, vr,
                                   np.array([3, 99, -1]), 8)
    want = orc.decode_attend_varlen(q, B, Hq, Hkv, ks, vs, np.array([40, 0, 0]), 40, kr, vr,
                                    np.array([3, 8, 0]), 8)
    assert np.array_equal(got, want)
    assert np.all(got[2] == 0.0) and np.all(np.abs(got[0]) > 0)
