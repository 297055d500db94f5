"""Pins for the oracle's bfloat16 paths (inputs and reconstructions stored as
bfloat16 instead of fp16; the packed store is the same).

  * the bfloat16 codec: all 65,536 patterns widen as torch's bfloat16 does,
    and narrowing agrees with torch's round-to-nearest-even conversion over
    whole fp32 exponents (every mantissa) and 4M random patterns;
  * hand-worked groups with dyadic values, whose codes and bfloat16
    reconstructions are exact by hand;
  * brute force: random groups against the exact-rational emulation in
    _exact.py with bfloat16 rounding (it shares no arithmetic with the C
    oracle), including values outside fp16's range;
  * the tensor flushes reduce to the group function on every group;
  * the bfloat16 attend equals torch's float64 scaled_dot_product_attention
    (a library routine) over the bfloat16 reconstruction of the store and
    the bfloat16 residual, and a single token returns its value.
"""
import numpy as np
import pytest
import torch

import _exact

D = 128


def _torch_bf16_to_f32(u16):
    return torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).float().numpy()


def _torch_f32_to_bf16(f32):
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_to_f32_all_65536(orc):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(allb)
    want = _torch_bf16_to_f32(allb)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("expo", [0, 1, 60, 126, 127, 128, 200, 254])
def test_f32_to_bf16_whole_exponents(orc, expo):
    """Every mantissa of one fp32 exponent, both signs (exponent 0 is the
    subnormals, 254 holds the overflow boundary)."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        bits = (np.uint32(sign) << np.uint32(31)) | (np.uint32(expo) << np.uint32(23)) | mant
        f = bits.view(np.float32)
        assert np.array_equal(orc.f32_to_bf16(f), _torch_f32_to_bf16(f))


def test_f32_to_bf16_random_patterns(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    fin = np.isfinite(f)
    assert np.array_equal(orc.f32_to_bf16(f[fin]), _torch_f32_to_bf16(f[fin]))


HAND = [
    # bits, inputs (exact in bfloat16), scale, codes, reconstruction bits
    (2, [0.0, 0.5, 1.5, 3.0], 1.0, [0, 0, 2, 3], [0x0000, 0x0000, 0x4000, 0x4040]),
    (4, [0.0, 15.0, 0.5, 1.5, 2.5, 3.5, 14.5], 1.0, [0, 15, 0, 2, 2, 4, 14],
     [0x0000, 0x4170, 0x0000, 0x4000, 0x4000, 0x4080, 0x4160]),
    (2, [-2.0, -0.5, 0.25, 1.0], 1.0, [0, 2, 2, 3], [0xC000, 0x0000, 0x0000, 0x3F80]),
    # beyond fp16's range: 2^20 .. 2^20 + 3 * 2^13, scale 2^13
    (2, [2.0 ** 20, 2.0 ** 20 + 2 ** 13, 2.0 ** 20 + 3 * 2 ** 13], 2.0 ** 13, [0, 1, 3],
     [0x4980, 0x4981, 0x4983]),
]


@pytest.mark.parametrize("row", HAND, ids=lambda r: f"b{r[0]}-{r[1][:2]}")
def test_hand_worked_bf16_groups(orc, row):
    bits, xs, scale, codes, recon = row
    xb = _torch_f32_to_bf16(np.array(xs, np.float32))
    assert np.array_equal(_torch_bf16_to_f32(xb), np.array(xs, np.float32))   # inputs are exact
    sc, ze, q, rec = orc.quantize_group(xb, bits, fmt="bf16")
    assert sc == np.float32(scale) and ze == np.float32(min(xs))
    assert q.tolist() == codes
    assert [int(v) for v in rec] == recon


def test_bf16_reconstruction_ties_round_to_even(orc):
    """With scale 2^12 = half a bfloat16 ulp at 2^20, code 1 lands exactly
    between 2^20 and 2^20 + 2^13 and code 3 between 2^20 + 2^13 and
    2^20 + 2^14: both ties go to the even encoding."""
    s, z = np.float32(2.0 ** 12), np.float32(2.0 ** 20)
    assert orc.dequantize_one(1, s, z, fmt="bf16") == 0x4980
    assert orc.dequantize_one(3, s, z, fmt="bf16") == 0x4982
    assert orc.dequantize_one(2, s, z, fmt="bf16") == 0x4981


@pytest.mark.parametrize("bits", [2, 4])
def test_random_bf16_groups_against_exact(orc, bits):
    rng = np.random.default_rng(100 + bits)
    for trial in range(300):
        n = int(rng.integers(1, 33))
        mag = 10.0 ** rng.uniform(-30, 30)          # far outside fp16's range too
        xs = (rng.standard_normal(n) * mag).astype(np.float32)
        xb = _torch_f32_to_bf16(xs)
        sc, ze, q, rec = orc.quantize_group(xb, bits, fmt="bf16")
        esc, eze, eq, erec = _exact.quantize_group([int(b) for b in xb], bits, fmt="bf16")
        assert np.float32(sc).view(np.uint32) == _exact.f32_bits(esc), trial
        assert np.float32(ze) == np.float32(float(eze)), trial
        assert q.tolist() == eq, trial
        assert [int(v) for v in rec] == erec, trial


def test_bf16_flushes_reduce_to_the_group_function(orc):
    rng = np.random.default_rng(3)
    BH, S = 2, 70                                  # a ragged last key group
    x = _torch_f32_to_bf16((rng.standard_normal((BH, S, D)) * 50).astype(np.float32))
    ks = orc.Store(orc.KEYS, BH, 96, D, 4)
    vs = orc.Store(orc.VALUES, BH, 96, D, 2)
    rk = orc.quantize_keys(x, ks, 0, fmt="bf16")
    rv = orc.quantize_values(x, vs, 0, fmt="bf16")
    for bh in range(BH):
        for g in range(3):
            s0, s1 = 32 * g, min(32 * g + 32, S)
            for d in (0, 5, 127):
                sc, ze, q, rec = orc.quantize_group(x[bh, s0:s1, d], 4, fmt="bf16")
                assert ks.scale[bh, g, d] == sc and ks.zero[bh, g, d] == ze
                assert np.array_equal(rk[bh, s0:s1, d], rec)
        for s in (0, 31, 69):
            for j in range(4):
                sc, ze, q, rec = orc.quantize_group(x[bh, s, 32 * j:32 * j + 32], 2, fmt="bf16")
                assert vs.scale[bh, s, j] == sc and vs.zero[bh, s, j] == ze
                assert np.array_equal(rv[bh, s, 32 * j:32 * j + 32], rec)
    assert np.array_equal(orc.dequantize(ks, 0, S, fmt="bf16"), rk)
    assert np.array_equal(orc.dequantize(vs, 0, S, fmt="bf16"), rv)


def _bf16_tensor(rng, shape, scale=1.0):
    return _torch_f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("bits", [4, 2])
def test_bf16_attend_matches_torch_sdpa(orc, bits):
    rng = np.random.default_rng(60 + bits)
    B, Hq, Hkv, nq, nr = 2, 8, 2, 70, 9
    BH = B * Hkv
    k = _bf16_tensor(rng, (BH, nq, D), 3.0)
    v = _bf16_tensor(rng, (BH, nq, D))
    kr = _bf16_tensor(rng, (BH, 16, D), 3.0)
    vr = _bf16_tensor(rng, (BH, 16, D))
    q = _bf16_tensor(rng, (B, Hq, D))
    ks = orc.Store(orc.KEYS, BH, 96, D, bits)
    vs = orc.Store(orc.VALUES, BH, 96, D, bits)
    orc.quantize_keys(k, ks, fmt="bf16", want_recon=False)
    orc.quantize_values(v, vs, fmt="bf16", want_recon=False)
    out = orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr, fmt="bf16")
    K = np.concatenate([orc.dequantize(ks, 0, nq, fmt="bf16"), kr[:, :nr]], axis=1)
    V = np.concatenate([orc.dequantize(vs, 0, nq, fmt="bf16"), vr[:, :nr]], axis=1)
    K = _torch_bf16_to_f32(K).astype(np.float64).reshape(B, Hkv, nq + nr, D)
    V = _torch_bf16_to_f32(V).astype(np.float64).reshape(B, Hkv, nq + nr, D)
    g = Hq // Hkv
    qt = torch.from_numpy(_torch_bf16_to_f32(q).astype(np.float64)).reshape(B, Hq, 1, D)
    want = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K).repeat_interleave(g, dim=1),
        torch.from_numpy(V).repeat_interleave(g, dim=1)).reshape(B, Hq, D).numpy()
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    # the same bit patterns read as fp16 give a different result: the format
    # reaches every input
    assert not np.allclose(orc.decode_attend(q, B, Hq, Hkv, ks, vs, nq, kr, vr, nr), want)


def test_bf16_attend_single_token_returns_its_value(orc):
    rng = np.random.default_rng(3)
    vr = _bf16_tensor(rng, (1, 1, D), 1e20)           # outside fp16's range
    kr = _bf16_tensor(rng, (1, 1, D))
    q = _bf16_tensor(rng, (1, 4, D))
    out = orc.decode_attend(q, 1, 4, 1, None, None, 0, kr, vr, 1, fmt="bf16")
    for h in range(4):
        assert np.array_equal(out[0, h], _torch_bf16_to_f32(vr[0, 0]).astype(np.float64))
