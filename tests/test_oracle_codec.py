"""Pins for the oracle's IEEE binary16 codec.

The oracle writes the codec from the format's definition; here it is checked
against two independent library implementations (torch's CPU converter and
numpy's), exhaustively wherever fp32 -> fp16 rounding actually happens.
"""
import numpy as np
import pytest
import torch


def _torch_f32_to_f16(f: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f).half().view(torch.int16).numpy().view(np.uint16)


def test_f16_to_f32_all_65536(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref_np = h.view(np.float16).astype(np.float32)
    ref_t = torch.from_numpy(h.view(np.int16)).view(torch.float16).float().numpy()
    nan = np.isnan(ref_np)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref_np[~nan].view(np.uint32))
    assert np.array_equal(got[~nan].view(np.uint32), ref_t[~nan].view(np.uint32))
    # spot values from the format's definition
    assert orc.f16_to_f32(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    assert orc.f16_to_f32(np.array([0x03FF], np.uint16))[0] == 1023 * 2.0 ** -24
    assert orc.f16_to_f32(np.array([0x0400], np.uint16))[0] == 2.0 ** -14
    assert orc.f16_to_f32(np.array([0x7BFF], np.uint16))[0] == 65504.0
    assert orc.f16_to_f32(np.array([0xC000], np.uint16))[0] == -2.0


def test_f16_roundtrip_all_finite(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    back = orc.f32_to_f16(orc.f16_to_f32(h))
    assert np.array_equal(back[finite], h[finite])


@pytest.mark.parametrize("sign", [0, 1])
def test_f32_to_f16_exhaustive_rounding_range(orc, sign):
    """Every fp32 whose biased exponent is 101..143, i.e. from below half the
    smallest fp16 subnormal (2^-25) to beyond the fp16 overflow threshold."""
    torch.set_num_threads(8)
    mism = 0
    chunk = 1 << 23  # one exponent's worth of mantissas
    for e in range(101, 144):
        base = (sign << 31) | (e << 23)
        bits = np.arange(base, base + chunk, dtype=np.uint64).astype(np.uint32)
        f = bits.view(np.float32)
        mism += int(np.count_nonzero(orc.f32_to_f16(f) != _torch_f32_to_f16(f)))
    assert mism == 0


def test_f32_to_f16_samples_elsewhere(orc):
    rng = np.random.default_rng(12345)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    got = orc.f32_to_f16(f)
    ref = _torch_f32_to_f16(f)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f32_to_f16_special_points(orc):
    cases = {
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7C00,          # the tie above the largest finite goes to inf
        float("inf"): 0x7C00,
        2.0 ** -24: 0x0001,
        2.0 ** -25: 0x0000,       # exact tie between 0 and the smallest subnormal
        1.5 * 2.0 ** -25: 0x0001,
        3 * 2.0 ** -25: 0x0002,   # tie between 1 and 2 subnormal quanta -> even
        1.0 + 2.0 ** -11: 0x3C00,  # tie between 1 and 1+2^-10 -> even (1)
        1.0 + 3 * 2.0 ** -11: 0x3C02,
        -0.0: 0x8000,
    }
    for v, want in cases.items():
        assert int(orc.f32_to_f16(np.array([v], np.float32))[0]) == want, v
