"""GPU parity of stores with binary16 scale and zero (KIVI_META_F16) against
the oracle's binary16-metadata variant: codes, scales, zeros (as binary16
bits) and reconstructions bit-exact for the flush and the dequantize, and the
uniform and variable-length attends within 2e-3 of the oracle's attend over
the same store.  Inputs span magnitudes from fp16 subnormals to 10, so that
scales round to binary16 subnormals or to 0 (the flush's exact path and its
clip) as well as to normal values (the fast path)."""
import numpy as np
import pytest
import torch

import oracle
from oracle_pool import pmap
from gpu_util import (CODE_SENTINEL, META_SENTINEL, assert_store_equal, assert_u16_equal, note, u16)
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128
KINDS = {"keys": kivi.KIVI_KEYS, "values": kivi.KIVI_VALUES}
SENTINEL16 = 0x7BFF
TOL = 2e-3


def _stores(kind, BH, cap, bits, G):
    k = KINDS[kind]
    st = kivi.Store(k, BH, cap, bits, group=G, meta="f16")
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    okind = oracle.KEYS if k == kivi.KIVI_KEYS else oracle.VALUES
    hs = oracle.Store(okind, BH, cap, D, bits, G, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL,
                      meta="f16")
    return st, hs


def _wide_range(BH, S, kind, seed):
    """fp16 [BH][S][128]: normal noise times a magnitude 10^U(-8, 1) per key
    group block (32 tokens x 1 channel) or per value block (1 token x 32
    channels), with some blocks constant and some all zero."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((BH, S, D))
    if kind == "keys":
        mag = 10.0 ** rng.uniform(-8, 1, size=(BH, (S + 31) // 32, 1, D))
        mag = np.repeat(mag, 32, axis=2).reshape(BH, -1, D)[:, :S]
    else:
        mag = 10.0 ** rng.uniform(-8, 1, size=(BH, S, D // 32, 1))
        mag = np.repeat(mag, 32, axis=3).reshape(BH, S, D)
    x = x * mag
    if S >= 4:
        x[:, 1, :] = 0.0                      # zero rows (constant value groups)
        x[:, :, 5] = 0.25                     # a constant channel (constant key groups)
    return torch.from_numpy(x.astype(np.float16)).cuda()


CASES = [
    # BH, S, cap, dst (keys: a multiple of G; values: any)
    (3, 101, 256, (128, 7)),
    (2, 64, 128, (0, 0)),
    (1, 1, 128, (0, 3)),
    (4, 300, 384, (0, 50)),
]


@pytest.mark.parametrize("inputs", ["kv", "wide"])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "BH%d-S%d" % (c[0], c[1]))
def test_flush_and_dequantize(case, G, kind, bits, inputs):
    BH, S, cap, (dst_k, dst_v) = case
    dst = (dst_k // G) * G if kind == "keys" else dst_v
    if dst + S > cap:
        pytest.skip("window past the store")
    seed = 12000 + G + S + bits
    if inputs == "kv":
        x = synth.kv_tensor(BH, S, keys=(kind == "keys"), seed=seed, device="cuda")
    else:
        x = _wide_range(BH, S, kind, seed)
    st, hs = _stores(kind, BH, cap, bits, G)
    recon_full = torch.full((BH, S + 8, D), SENTINEL16, dtype=torch.int16, device="cuda").view(torch.float16)
    note(f"binary16 metadata {inputs} flush {kind} G={G} bits={bits} BH={BH} S={S} cap={cap} dst={dst}")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, dst, recon_full[:, :S])
    torch.cuda.synchronize()
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    hrec = ofn(u16(x), hs, dst, want_recon=True)
    what = f"meta16 {inputs} G={G} {kind} bits={bits} S={S} dst={dst}"
    assert_store_equal(st, hs, what=what)
    r = u16(recon_full)
    assert_u16_equal(r[:, :S], hrec, what + " recon")
    assert np.all(r[:, S:] == SENTINEL16), "recon written past the window"
    # without the fused reconstruction: same store
    st2, _ = _stores(kind, BH, cap, bits, G)
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st2, dst)
    out = kivi.dequantize(st, dst, S)
    torch.cuda.synchronize()
    assert_store_equal(st2, hs, what=what + " (no recon)")
    assert_u16_equal(u16(out), hrec, what + " dequantize")


def test_wide_inputs_reach_the_slow_scales():
    """The wide-range inputs do produce binary16 scales that are subnormal or
    0 for non-constant groups, so the tests above cover the exact path."""
    x = _wide_range(2, 128, "keys", 5)
    hs = oracle.Store(oracle.KEYS, 2, 128, D, 4, 32, meta="f16")
    oracle.quantize_keys(u16(x), hs, 0, want_recon=False)
    xs = x.float().cpu().numpy().reshape(2, 4, 32, D)
    rng = xs.max(axis=2) - xs.min(axis=2)
    sub = (hs.scale < 2.0 ** -14) & (rng > 0)
    assert np.count_nonzero(sub & (hs.scale > 0)) > 10
    assert np.count_nonzero(sub & (hs.scale == 0)) > 10


ATTEND = [
    # B, Hq, Hkv, n_quant, n_res, bits
    (2, 32, 8, 1000, 37, 4),
    (1, 32, 8, 4096 + 64, 128, 4),
    (3, 64, 8, 300, 5, 2),
    (4, 16, 16, 640, 0, 4),
]


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("case", ATTEND, ids=lambda c: "B%d-Hq%d-nq%d-nr%d-b%d" % (c[0], c[1], c[3], c[4], c[5]))
def test_attend(case, G):
    B, Hq, Hkv, nq, nr, bits = case
    BH = B * Hkv
    cap = ((nq + G - 1) // G) * G
    seed = 13100 + nq + G
    kx = synth.kv_tensor(BH, nq, keys=True, seed=seed, device="cuda")
    vx = synth.kv_tensor(BH, nq, keys=False, seed=seed, device="cuda")
    kr = synth.residual(BH, max(nr, 1), keys=True, seed=seed, device="cuda")
    vr = synth.residual(BH, max(nr, 1), keys=False, seed=seed, device="cuda")
    q = synth.query(B, Hq, seed=seed, device="cuda")
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, bits, group=G, meta="f16")
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, bits, group=G, meta="f16")
    note(f"attend over binary16-metadata G={G} stores B={B} Hq={Hq} n_quant={nq} n_res={nr} bits={bits}")
    kivi.quantize_keys(kx, ks, 0)
    kivi.quantize_values(vx, vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr)
    # varlen: every sequence its own length
    rng = np.random.default_rng(seed)
    nq_h = rng.integers(0, nq + 1, size=B).astype(np.int32)
    nr_h = rng.integers(0, nr + 1, size=B).astype(np.int32)
    nr_h[(nq_h + nr_h) == 0] = max(nr, 0)
    nq_h[(nq_h + nr_h) == 0] = nq
    out_v = kivi.decode_attend_varlen(q, ks, vs, torch.from_numpy(nq_h).cuda(), nq, kr, vr,
                                      torch.from_numpy(nr_h).cuda(), nr)
    torch.cuda.synchronize()
    hk = oracle.Store(oracle.KEYS, BH, cap, D, bits, G, meta="f16")
    hv = oracle.Store(oracle.VALUES, BH, cap, D, bits, G, meta="f16")
    oracle.quantize_keys(u16(kx), hk, 0, want_recon=False)
    oracle.quantize_values(u16(vx), hv, 0, want_recon=False)
    assert_store_equal(ks, hk, what="keys")
    assert_store_equal(vs, hv, what="values")
    ref = oracle.decode_attend(u16(q), B, Hq, Hkv, hk, hv, nq, u16(kr), u16(vr), nr)
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    assert err <= TOL, f"max-abs error {err:.3e}"
    ref_v = oracle.decode_attend_varlen(u16(q), B, Hq, Hkv, hk, hv, nq_h, nq, u16(kr), u16(vr),
                                        nr_h, nr)
    err = float(np.max(np.abs(out_v.cpu().numpy().astype(np.float64) - ref_v)))
    assert err <= TOL, f"varlen max-abs error {err:.3e}"


def test_full_size_attend():
    """The measured shape (32 sequences x 32 query heads over 8 kv heads,
    16384 store tokens + 128 residual, 4-bit, groups of 32): every sequence
    against the oracle."""
    B, Hq, Hkv, nq, nr = 32, 32, 8, 16384, 128
    BH = B * Hkv
    seed = 777
    kx = synth.kv_tensor(BH, nq, keys=True, seed=seed, device="cuda")
    vx = synth.kv_tensor(BH, nq, keys=False, seed=seed + 1, device="cuda")
    kr = synth.residual(BH, nr, keys=True, seed=seed, device="cuda")
    vr = synth.residual(BH, nr, keys=False, seed=seed, device="cuda")
    q = synth.query(B, Hq, seed=seed, device="cuda")
    ks = kivi.Store(kivi.KIVI_KEYS, BH, nq, 4, meta="f16")
    vs = kivi.Store(kivi.KIVI_VALUES, BH, nq, 4, meta="f16")
    note("attend binary16 metadata full size B=32 n_quant=16384")
    kivi.quantize_keys(kx, ks, 0)
    kivi.quantize_values(vx, vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    hkx, hvx, hkr, hvr, hq = u16(kx), u16(vx), u16(kr), u16(vr), u16(q)

    def one(b):
        sl = slice(b * Hkv, (b + 1) * Hkv)
        hk = oracle.Store(oracle.KEYS, Hkv, nq, D, 4, 32, meta="f16")
        hv = oracle.Store(oracle.VALUES, Hkv, nq, D, 4, 32, meta="f16")
        oracle.quantize_keys(hkx[sl], hk, 0, want_recon=False)
        oracle.quantize_values(hvx[sl], hv, 0, want_recon=False)
        return oracle.decode_attend(hq[b:b + 1], 1, Hq, Hkv, hk, hv, nq, hkr[sl], hvr[sl], nr)[0]
    for b, ref in enumerate(pmap(one, range(B))):
        err = float(np.max(np.abs(got[b] - ref)))
        assert err <= TOL, f"sequence {b}: max-abs error {err:.3e}"


@pytest.mark.parametrize("kind", ["keys", "values"])
def test_hand_worked_groups_on_gpu(kind):
    """Every hand-worked group of tests/golden/meta16_groups.txt as a real
    group of the flush (a key channel's 32 tokens, or a token's first value
    group, padded with copies of its minimum): the stored binary16 scale and
    zero, the codes and the fused reconstruction equal the fixture's values.
    The midpoint_scale row is a scale whose binary32 value is a binary16
    tie, where a single rounding straight to binary16 goes the other way."""
    from golden_io import hexes, ints, rows
    for r in rows("meta16_groups.txt"):
        name, bits, xs = r[0], int(r[1]), hexes(r[2])
        want_s, want_z = hexes(r[3])[0], hexes(r[4])[0]
        want_q, want_rec = ints(r[5]), hexes(r[6])
        n = len(xs)
        mn = min(xs, key=lambda b: float(np.array([b], np.uint16).view(np.float16)[0]))
        grp = np.array(xs + [mn] * (32 - n), np.uint16)
        x = np.zeros((1, 32, D), np.uint16)
        if kind == "keys":
            x[0, :, 0] = grp                    # channel 0, tokens 0..31
        else:
            x[0, 0, :32] = grp                  # token 0, channels 0..31
        x_dev = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
        st, hs = _stores(kind, 1, 32, bits, 32)
        rec = torch.empty_like(x_dev)
        note(f"hand-worked binary16 group {name} as {kind}")
        (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x_dev, st, 0, rec)
        torch.cuda.synchronize()
        s = int(st.scale.view(torch.int16)[0, 0, 0]) & 0xFFFF
        z = int(st.zero.view(torch.int16)[0, 0, 0]) & 0xFFFF
        assert (s, z) == (want_s, want_z), f"{name} {kind}: scale/zero {s:#06x}/{z:#06x}"
        words = st.codes.cpu().numpy().view(np.uint32)[0]
        r16 = u16(rec)[0]
        per_word = 32 // bits
        for i in range(n):
            t, c = (i, 0) if kind == "keys" else (0, i)
            q = (int(words[t, c // per_word]) >> (bits * (c % per_word))) & ((1 << bits) - 1)
            assert q == want_q[i], f"{name} {kind}: code {i} is {q}, fixture {want_q[i]}"
            assert int(r16[t, c]) == want_rec[i], f"{name} {kind}: recon {i} {int(r16[t, c]):#06x}"
