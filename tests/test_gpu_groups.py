"""GPU parity of the flush and dequantize with groups of 64 and 128 tokens
(keys) or channels (values) against the oracle: codes, scales, zeros and the
fp16 or bfloat16 reconstructions bit-exact, every output buffer sentinel-
filled so whole-array comparisons also check the write window."""
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


def _stores(kind, BH, cap, bits, G):
    k = KINDS[kind]
    st = kivi.Store(k, BH, cap, bits, group=G)
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    okind = oracle.KEYS if k == kivi.KIVI_KEYS else oracle.VALUES
    hs = oracle.Store(okind, BH, cap, D, bits, G, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL)
    return st, hs


CASES = [
    # BH, S as a multiple of G plus a tail, cap in groups, dst in groups (keys) / tokens (values)
    (3, (2, 37), 4, (1, 5)),
    (2, (1, 0), 2, (0, 0)),
    (1, (0, 1), 1, (0, 3)),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "BH%d-S%dG+%d" % (c[0], c[1][0], c[1][1]))
def test_group_sizes(case, G, kind, bits, fmt):
    BH, (ng, tail), cap_g, (dst_g, dst_v) = case
    S = ng * G + tail
    cap = cap_g * G
    dst = dst_g * G if kind == "keys" else dst_v
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    x = synth.kv_tensor(BH, S, keys=(kind == "keys"), seed=8000 + G + S, device="cuda", dtype=dtype)
    st, hs = _stores(kind, BH, cap, bits, G)
    recon_full = torch.full((BH, S + 8, D), SENTINEL16, dtype=torch.int16, device="cuda").view(dtype)
    note(f"group {G} {fmt} flush {kind} bits={bits} BH={BH} S={S} cap={cap} dst={dst}")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, dst, recon_full[:, :S])
    torch.cuda.synchronize()
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    hrec = ofn(u16(x), hs, dst, want_recon=True, fmt=fmt)
    what = f"G={G} {fmt} {kind} bits={bits} S={S} dst={dst}"
    assert_store_equal(st, hs, what=what)
    r = u16(recon_full)
    assert_u16_equal(r[:, :S], hrec, what + " recon")
    assert np.all(r[:, S:] == SENTINEL16), "recon written past the window"
    out = kivi.dequantize(st, dst, S, dtype=dtype)
    torch.cuda.synchronize()
    assert_u16_equal(u16(out), hrec, what + " dequantize")


def test_dequantize_ranges_inside_wide_key_groups():
    """Dequantize windows that start inside a key group of 128 and end inside
    another one: every row reads its own group's scale and zero."""
    BH, G, S = 2, 128, 384
    x = synth.kv_tensor(BH, S, keys=True, seed=9, device="cuda")
    st, hs = _stores("keys", BH, S, 4, G)
    kivi.quantize_keys(x, st, 0)
    oracle.quantize_keys(u16(x), hs, 0, want_recon=False)
    for t0, n in ((5, 40), (96, 64), (120, 200), (0, 384)):
        note(f"dequantize G=128 tokens [{t0}, {t0 + n})")
        out = kivi.dequantize(st, t0, n)
        torch.cuda.synchronize()
        assert_u16_equal(u16(out), oracle.dequantize(hs, t0, n), f"[{t0}, {t0 + n})")


ATTEND = [
    # B, Hq, Hkv, n_quant, n_res, bits
    (2, 32, 8, 1000, 37, 4),
    (1, 32, 8, 4096 + 64, 128, 4),
    (3, 64, 8, 300, 5, 2),
    (2, 32, 8, 0, 64, 4),
]


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("case", ATTEND, ids=lambda c: "B%d-Hq%d-nq%d-nr%d-b%d" % (c[0], c[1], c[3], c[4], c[5]))
def test_attend_over_wide_group_stores(case, G):
    B, Hq, Hkv, nq, nr, bits = case
    BH = B * Hkv
    cap = max(G, ((nq + G - 1) // G) * G)
    seed = 9100 + nq + G
    kx = synth.kv_tensor(BH, max(nq, 1), keys=True, seed=seed, device="cuda")[:, :nq]
    vx = synth.kv_tensor(BH, max(nq, 1), keys=False, seed=seed, device="cuda")[:, :nq]
    kr = synth.residual(BH, max(nr, 1), keys=True, seed=seed, device="cuda")
    vr = synth.residual(BH, max(nr, 1), keys=False, seed=seed, device="cuda")
    q = synth.query(B, Hq, seed=seed, device="cuda")
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, bits, group=G)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, bits, group=G)
    note(f"attend over G={G} stores B={B} Hq={Hq} n_quant={nq} n_res={nr} bits={bits}")
    if nq:
        kivi.quantize_keys(kx, ks, 0)
        kivi.quantize_values(vx, vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr)
    nq_t = torch.full((B,), nq, dtype=torch.int32, device="cuda")
    nr_t = torch.full((B,), nr, dtype=torch.int32, device="cuda")
    out_v = kivi.decode_attend_varlen(q, ks, vs, nq_t, nq, kr, vr, nr_t, nr)
    torch.cuda.synchronize()
    hk = oracle.Store(oracle.KEYS, BH, cap, D, bits, G)
    hv = oracle.Store(oracle.VALUES, BH, cap, D, bits, G)
    if nq:
        oracle.quantize_keys(u16(kx), hk, 0, want_recon=False)
        oracle.quantize_values(u16(vx), hv, 0, want_recon=False)
    ref = oracle.decode_attend(u16(q), B, Hq, Hkv, hk, hv, nq, u16(kr), u16(vr), nr)
    for got in (out, out_v):
        err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - ref)))
        assert err <= 2e-3, f"max-abs error {err:.3e}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("Dh", [64, 256])
@pytest.mark.parametrize("shape", [(3, 101, 160, 32, 7), (1, 64, 64, 0, 0), (2, 1, 64, 32, 1)],
                         ids=lambda c: "BH%d-S%d-dst%d" % (c[0], c[1], c[3]))
def test_other_head_dims(shape, Dh, kind, bits, fmt):
    """head_dim 64 and 256 with groups of 32: flush (with fused
    reconstruction) and dequantize bit-exact against the oracle."""
    BH, S, cap, dst_k, dst_v = shape
    dst = dst_k if kind == "keys" else dst_v
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    x = synth.kv_tensor(BH, S, Dh, keys=(kind == "keys"), seed=8500 + Dh + S, device="cuda", dtype=dtype)
    k = KINDS[kind]
    st = kivi.Store(k, BH, cap, bits, head_dim=Dh)
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    okind = oracle.KEYS if k == kivi.KIVI_KEYS else oracle.VALUES
    hs = oracle.Store(okind, BH, cap, Dh, bits, 32, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL)
    recon_full = torch.full((BH, S + 8, Dh), SENTINEL16, dtype=torch.int16, device="cuda").view(dtype)
    note(f"head_dim {Dh} {fmt} flush {kind} bits={bits} BH={BH} S={S} cap={cap} dst={dst}")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, dst, recon_full[:, :S])
    torch.cuda.synchronize()
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    hrec = ofn(u16(x), hs, dst, want_recon=True, fmt=fmt)
    what = f"D={Dh} {fmt} {kind} bits={bits} S={S} dst={dst}"
    assert_store_equal(st, hs, what=what)
    r = u16(recon_full)
    assert_u16_equal(r[:, :S], hrec, what + " recon")
    assert np.all(r[:, S:] == SENTINEL16), "recon written past the window"
    out = kivi.dequantize(st, dst, S, dtype=dtype)
    torch.cuda.synchronize()
    assert_u16_equal(u16(out), hrec, what + " dequantize")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("Dh", [16, 32, 48, 80, 96, 112, 144, 160, 176, 192, 208, 224, 240])
@pytest.mark.parametrize("shape", [(3, 101, 160, 32, 7), (2, 64, 64, 0, 0), (1, 1, 64, 32, 1)],
                         ids=lambda c: "BH%d-S%d-dst%d" % (c[0], c[1], c[3]))
def test_other_head_dims(shape, Dh, kind, bits, fmt):
    """Every admitted head_dim other than 64, 128 and 256: a row of
    head_dim/8 chunks in 8, 16 or 32 lanes, the lanes past its last chunk
    idle (a token's last value group has 16 channels when 32 does not divide
    head_dim): flush with fused reconstruction, and dequantize, bit-exact
    against the oracle, sentinel-filled outputs checking the write window."""
    BH, S, cap, dst_k, dst_v = shape
    dst = dst_k if kind == "keys" else dst_v
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    x = synth.kv_tensor(BH, S, Dh, keys=(kind == "keys"), seed=8700 + Dh + S, device="cuda", dtype=dtype)
    k = KINDS[kind]
    st = kivi.Store(k, BH, cap, bits, head_dim=Dh)
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    okind = oracle.KEYS if k == kivi.KIVI_KEYS else oracle.VALUES
    hs = oracle.Store(okind, BH, cap, Dh, bits, 32, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL)
    recon_full = torch.full((BH, S + 8, Dh), SENTINEL16, dtype=torch.int16, device="cuda").view(dtype)
    note(f"head_dim {Dh} {fmt} flush {kind} bits={bits} BH={BH} S={S} cap={cap} dst={dst}")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, dst, recon_full[:, :S])
    torch.cuda.synchronize()
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    hrec = ofn(u16(x), hs, dst, want_recon=True, fmt=fmt)
    what = f"D={Dh} {fmt} {kind} bits={bits} S={S} dst={dst}"
    assert_store_equal(st, hs, what=what)
    r = u16(recon_full)
    assert_u16_equal(r[:, :S], hrec, what + " recon")
    assert np.all(r[:, S:] == SENTINEL16), "recon written past the window"
    out = kivi.dequantize(st, dst, S, dtype=dtype)
    torch.cuda.synchronize()
    assert_u16_equal(u16(out), hrec, what + " dequantize")
    # the same flush without the fused reconstruction writes the same store
    st2 = kivi.Store(k, BH, cap, bits, head_dim=Dh)
    st2.codes.fill_(CODE_SENTINEL)
    st2.scale.fill_(META_SENTINEL)
    st2.zero.fill_(META_SENTINEL)
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st2, dst)
    torch.cuda.synchronize()
    assert_store_equal(st2, hs, what=what + " (no recon)")


ATTEND64 = [
    # B, Hq, Hkv, n_quant, n_res, bits
    (2, 32, 8, 1000, 37, 4),
    (1, 16, 2, 4096 + 64, 128, 4),
    (3, 64, 8, 300, 5, 2),
    (2, 32, 8, 0, 64, 4),
    (4, 8, 8, 640, 0, 2),
    (2, 8, 1, 2048, 3, 4),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", ATTEND64, ids=lambda c: "B%d-Hq%d-Hkv%d-nq%d-nr%d-b%d" % c)
def test_attend_head_dim_64(case, fmt):
    """The decode attends (uniform and variable-length) at head_dim 64 with
    groups of 32, fp16 and bfloat16, against the oracle (tolerance 2e-3 in
    both formats)."""
    B, Hq, Hkv, nq, nr, bits = case
    Dh = 64
    BH = B * Hkv
    cap = max(32, ((nq + 31) // 32) * 32)
    seed = 9300 + nq + nr + bits
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    kx = synth.kv_tensor(BH, max(nq, 1), Dh, keys=True, seed=seed, device="cuda", dtype=dtype)[:, :nq]
    vx = synth.kv_tensor(BH, max(nq, 1), Dh, keys=False, seed=seed, device="cuda", dtype=dtype)[:, :nq]
    kr = synth.residual(BH, max(nr, 1), Dh, keys=True, seed=seed, device="cuda").to(dtype)
    vr = synth.residual(BH, max(nr, 1), Dh, keys=False, seed=seed, device="cuda").to(dtype)
    q = synth.query(B, Hq, Dh, seed=seed, device="cuda").to(dtype)
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, bits, head_dim=Dh)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, bits, head_dim=Dh)
    note(f"attend head_dim 64 {fmt} B={B} Hq={Hq} Hkv={Hkv} n_quant={nq} n_res={nr} bits={bits}")
    if nq:
        kivi.quantize_keys(kx.contiguous(), ks, 0)
        kivi.quantize_values(vx.contiguous(), vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr)
    rng = np.random.default_rng(seed)
    nq_h = rng.integers(0, nq + 1, size=B).astype(np.int32)
    nr_h = rng.integers(0, nr + 1, size=B).astype(np.int32)
    empty = (nq_h + nr_h) == 0
    nq_h[empty], nr_h[empty] = nq, nr
    out_v = kivi.decode_attend_varlen(q, ks, vs, torch.from_numpy(nq_h).cuda(), nq, kr, vr,
                                      torch.from_numpy(nr_h).cuda(), nr)
    torch.cuda.synchronize()
    hk = oracle.Store(oracle.KEYS, BH, cap, Dh, bits, 32)
    hv = oracle.Store(oracle.VALUES, BH, cap, Dh, bits, 32)
    if nq:
        oracle.quantize_keys(u16(kx), hk, 0, want_recon=False, fmt=fmt)
        oracle.quantize_values(u16(vx), hv, 0, want_recon=False, fmt=fmt)
    tol = 2e-3
    ref = oracle.decode_attend(u16(q), B, Hq, Hkv, hk, hv, nq, u16(kr), u16(vr), nr, fmt=fmt)
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    print(f"{case} {fmt}: max-abs error {err:.2e}")
    assert err <= tol, f"max-abs error {err:.3e}"
    ref_v = oracle.decode_attend_varlen(u16(q), B, Hq, Hkv, hk, hv, nq_h, nq, u16(kr), u16(vr),
                                        nr_h, nr, fmt=fmt)
    err = float(np.max(np.abs(out_v.cpu().numpy().astype(np.float64) - ref_v)))
    assert err <= tol, f"varlen max-abs error {err:.3e}"


ATTEND_CASES = [
    # B, Hq, Hkv, n_quant, n_res, bits
    (2, 16, 8, 300, 37, 4),
    (1, 8, 2, 1000, 5, 2),
    (2, 8, 8, 0, 40, 4),
    (3, 4, 1, 200, 0, 4),
]
# plans the small cases above never reach: several steps per wave with a wave
# that runs from the store into the residual window, and a single sequence
# with eight query heads per kv head split 65 ways (the 16-wave combine)
ATTEND_PLANS = [
    (4, 32, 8, 2048, 128, 4),
    (1, 8, 1, 2048, 5, 4),
]
# every admitted head_dim but 128: 64 and 256 on their own MFMA geometry, the
# others padded to the next of 64, 128 and 256
OTHER_DIMS = [16, 32, 48, 64, 80, 96, 112, 144, 160, 176, 192, 208, 224, 240, 256]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Dh", [256, 96, 48, 176])
@pytest.mark.parametrize("case", ATTEND_PLANS, ids=lambda c: "B%d-Hq%d-Hkv%d-nq%d-nr%d-b%d" % c)
def test_attend_other_head_dim_plans(case, Dh, fmt):
    test_attend_other_head_dims(case, Dh, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Dh", OTHER_DIMS)
@pytest.mark.parametrize("case", ATTEND_CASES, ids=lambda c: "B%d-Hq%d-Hkv%d-nq%d-nr%d-b%d" % c)
def test_attend_other_head_dims(case, Dh, fmt):
    """The decode attends at head_dim 256 (16 PV accumulators per lane) and
    at the head_dims padded onto the 64-, 128- or 256-channel MFMA geometry
    (the channels past head_dim dequantized with zero scale and zero, zero
    queries and residual rows there, and never stored); groups of 32, held
    to 2e-3 in both formats; uniform and variable-length against the
    oracle."""
    B, Hq, Hkv, nq, nr, bits = case
    BH = B * Hkv
    cap = max(32, ((nq + 31) // 32) * 32)
    seed = 9500 + Dh + nq + nr
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    kx = synth.kv_tensor(BH, max(nq, 1), Dh, keys=True, seed=seed, device="cuda", dtype=dtype)[:, :nq]
    vx = synth.kv_tensor(BH, max(nq, 1), Dh, keys=False, seed=seed, device="cuda", dtype=dtype)[:, :nq]
    kr = synth.residual(BH, max(nr, 1), Dh, keys=True, seed=seed, device="cuda").to(dtype)
    vr = synth.residual(BH, max(nr, 1), Dh, keys=False, seed=seed, device="cuda").to(dtype)
    q = synth.query(B, Hq, Dh, seed=seed, device="cuda").to(dtype)
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, bits, head_dim=Dh)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, bits, head_dim=Dh)
    note(f"attend head_dim {Dh} {fmt} B={B} Hq={Hq} Hkv={Hkv} n_quant={nq} n_res={nr} bits={bits}")
    if nq:
        kivi.quantize_keys(kx.contiguous(), ks, 0)
        kivi.quantize_values(vx.contiguous(), vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr)
    rng = np.random.default_rng(seed)
    nq_h = rng.integers(0, nq + 1, size=B).astype(np.int32)
    nr_h = rng.integers(0, nr + 1, size=B).astype(np.int32)
    empty = (nq_h + nr_h) == 0
    nq_h[empty], nr_h[empty] = nq, nr
    out_v = kivi.decode_attend_varlen(q, ks, vs, torch.from_numpy(nq_h).cuda(), nq, kr, vr,
                                      torch.from_numpy(nr_h).cuda(), nr)
    torch.cuda.synchronize()
    hk = oracle.Store(oracle.KEYS, BH, cap, Dh, bits, 32)
    hv = oracle.Store(oracle.VALUES, BH, cap, Dh, bits, 32)
    if nq:
        oracle.quantize_keys(u16(kx), hk, 0, want_recon=False, fmt=fmt)
        oracle.quantize_values(u16(vx), hv, 0, want_recon=False, fmt=fmt)
    ref = oracle.decode_attend(u16(q), B, Hq, Hkv, hk, hv, nq, u16(kr), u16(vr), nr, fmt=fmt)
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    print(f"{case} D={Dh} {fmt}: max-abs error {err:.2e}")
    assert err <= 2e-3, f"max-abs error {err:.3e}"
    ref_v = oracle.decode_attend_varlen(u16(q), B, Hq, Hkv, hk, hv, nq_h, nq, u16(kr), u16(vr),
                                        nr_h, nr, fmt=fmt)
    err = float(np.max(np.abs(out_v.cpu().numpy().astype(np.float64) - ref_v)))
    assert err <= 2e-3, f"varlen max-abs error {err:.3e}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("Dh", [256, 96])
def test_attend_head_dims_at_the_bench_shape(Dh, fmt, bits):
    """head_dims 256 and 96 (padded to 128) at the bench's B=32 x 2048 + 128
    shape (32 query heads over 8 kv heads, several steps per wave): sampled
    sequences against the oracle within 2e-3."""
    B, Hq, Hkv, nq, nr = 32, 32, 8, 2048, 128
    BH = B * Hkv
    seed = 9700 + bits + Dh
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    kx = synth.kv_tensor(BH, nq, Dh, keys=True, seed=seed, device="cuda", dtype=dtype)
    vx = synth.kv_tensor(BH, nq, Dh, keys=False, seed=seed, device="cuda", dtype=dtype)
    kr = synth.residual(BH, nr, Dh, keys=True, seed=seed, device="cuda").to(dtype)
    vr = synth.residual(BH, nr, Dh, keys=False, seed=seed, device="cuda").to(dtype)
    q = synth.query(B, Hq, Dh, seed=seed, device="cuda").to(dtype)
    ks = kivi.Store(kivi.KIVI_KEYS, BH, nq, bits, head_dim=Dh)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, nq, bits, head_dim=Dh)
    note(f"attend head_dim {Dh} {fmt} bits={bits} B={B} S_kv={nq}+{nr}")
    kivi.quantize_keys(kx, ks, 0)
    kivi.quantize_values(vx, vs, 0)
    out = kivi.decode_attend(q, ks, vs, nq, kr, vr, nr).cpu().numpy()
    hq, hkx, hvx, hkr, hvr = u16(q), u16(kx), u16(vx), u16(kr), u16(vr)

    def one(b):
        sl = slice(b * Hkv, (b + 1) * Hkv)
        hk = oracle.Store(oracle.KEYS, Hkv, nq, Dh, bits, 32)
        hv = oracle.Store(oracle.VALUES, Hkv, nq, Dh, bits, 32)
        oracle.quantize_keys(hkx[sl], hk, 0, want_recon=False, fmt=fmt)
        oracle.quantize_values(hvx[sl], hv, 0, want_recon=False, fmt=fmt)
        return oracle.decode_attend(hq[b:b + 1], 1, Hq, Hkv, hk, hv, nq, hkr[sl], hvr[sl], nr, fmt=fmt)[0]
    samples = [0, 13, 31]
    for b, ref in zip(samples, pmap(one, samples)):
        err = float(np.max(np.abs(out[b].astype(np.float64) - ref)))
        assert err <= 2e-3, f"sequence {b}: max-abs error {err:.3e}"
