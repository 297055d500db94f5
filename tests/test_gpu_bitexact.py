"""Bit-exactness of the flush and dequantize where it is hardest to keep.

* Near-tie stress: tensors whose every quantization group holds 30 elements
  with a binary32 quotient within 2^-12 of a half-integer (tests/near_ties.py;
  exact ties included), over a million such elements per case, for keys and
  values, 4 and 2 bits, fp16 and bfloat16 inputs and binary16 scale/zero.
  These are the elements a reciprocal code or a rounding shortcut gets one
  off; the kernels' near-tie fallback must catch every one.
* A sweep of 300 seeded flush configurations over every store geometry and
  format the library takes (kind, bits, head_dim, group size, input format,
  scale/zero format, slab count, ragged lengths, write offsets, strided
  inputs, fused reconstruction, input magnitudes from subnormal to huge),
  each compared whole with the oracle: the pages' own bar is a 300-of-300
  bit-exact parity sweep ([Metal post] "Three ways to be off by one bit").

Codes, scales, zeros and 16-bit reconstructions (fused, and from the
dequantize kernel) are compared bit for bit; every output buffer starts
sentinel-filled, so the whole-array comparison also checks the write window.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (CODE_SENTINEL, META_SENTINEL, assert_store_equal, assert_u16_equal, note,
                      u16)
from near_ties import as_keys, as_values, near_tie_groups
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KINDS = {"keys": kivi.KIVI_KEYS, "values": kivi.KIVI_VALUES}
SENT16 = {"f16": 0x7BFF, "bf16": 0x7F7F}      # largest finite values: never a reconstruction here


def _run_both(kind, x_dev, bits, D, G, meta, cap, dst, with_recon, what):
    """One flush (and dequantize of its window) on both sides, compared whole."""
    BH, S, _ = x_dev.shape
    fmt = "bf16" if x_dev.dtype == torch.bfloat16 else "f16"
    k = KINDS[kind]
    st = kivi.Store(k, BH, cap, bits, group=G, head_dim=D, meta=meta)
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    recon_full = torch.full((BH, S + 8, D), SENT16[fmt], dtype=torch.int16,
                            device="cuda").view(x_dev.dtype)
    note(what)
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(
        x_dev, st, dst, recon_full[:, :S] if with_recon else None)
    out = kivi.dequantize(st, dst, S, dtype=x_dev.dtype) if S else None
    torch.cuda.synchronize()
    okind = oracle.KEYS if kind == "keys" else oracle.VALUES
    hs = oracle.Store(okind, BH, cap, D, bits, G, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL,
                      meta=meta)
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    hrec = ofn(np.ascontiguousarray(u16(x_dev)), hs, dst, want_recon=True, fmt=fmt)
    assert_store_equal(st, hs, what=what)
    r = u16(recon_full)
    if with_recon:
        assert_u16_equal(r[:, :S], hrec, what + " recon")
        assert np.all(r[:, S:] == SENT16[fmt]), what + ": recon written past the window"
    else:
        assert np.all(r == SENT16[fmt]), what + ": recon written without being asked"
    if S:
        assert_u16_equal(u16(out), hrec, what + " dequantize")


NEAR_CASES = [
    # bits, input format, scale/zero format
    (4, "f16", "f32"), (2, "f16", "f32"), (4, "f16", "f16"), (2, "f16", "f16"),
    (4, "bf16", "f32"), (2, "bf16", "f32"),
]


@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("case", NEAR_CASES, ids=lambda c: "b%d-%s-meta%s" % c)
def test_near_tie_stress(kind, case):
    bits, fmt, meta = case
    BH, S, D = 4, 2176, 128                     # 34816 key groups / value groups
    n_groups = BH * S * D // 32
    groups, n_near = near_tie_groups(n_groups, bits, seed=100 + bits + 7 * len(fmt + meta), fmt=fmt,
                                     meta=meta)
    assert n_near >= 10 ** 6
    xs = as_keys(groups, BH, S, D) if kind == "keys" else as_values(groups, BH, S, D)
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    x_dev = torch.from_numpy(xs.view(np.int16)).cuda().view(dtype)
    _run_both(kind, x_dev, bits, D, 32, meta, S, 0, True,
              f"near-tie stress {kind} bits={bits} {fmt} meta={meta}: {n_near} near-tie elements")


# ------------------------------------------------------------------ sweep
GEOMETRIES = [(128, 32), (128, 64), (128, 128), (64, 32), (256, 32),
              (16, 32), (48, 32), (80, 32), (96, 32), (112, 32), (144, 32), (160, 32),
              (192, 32), (208, 32), (240, 32)]
MAGNITUDES = {"f16": [1.0, 1.0, 1.0, 1e-3, 1e-5, 60.0],
              "bf16": [1.0, 1.0, 1e-3, 1e-30, 1e-38, 1e30]}


def sweep_configs(n=300, seed=300):
    rng = np.random.default_rng(seed)
    cfgs = []
    for i in range(n):
        kind = ("keys", "values")[i % 2]
        # head_dim 128 (the pages' geometry, every group size) in 40% of them
        g = rng.integers(3) if rng.random() < 0.4 else rng.integers(3, len(GEOMETRIES))
        D, G = GEOMETRIES[g]
        fmt = ("f16", "bf16")[rng.integers(2)]
        meta = "f16" if (fmt == "f16" and D == 128 and rng.random() < 0.5) else "f32"
        bits = (4, 2)[rng.integers(2)]
        BH = int(rng.integers(1, 7))
        S = int(rng.choice([rng.integers(1, 40), rng.integers(1, 5) * G, rng.integers(40, 700)]))
        if kind == "keys":
            dst = int(rng.integers(0, 4)) * G
        else:
            dst = int(rng.integers(0, 100))
        # capacity: whole groups, so every slab stride is whole 16-byte units
        cap = -(-(dst + S + int(rng.integers(0, 2 * G))) // G) * G
        pad = int(rng.choice([0, 0, rng.integers(1, 40)]))
        mag = float(rng.choice(MAGNITUDES[fmt]))
        recon = bool(rng.random() < 0.6)
        cfgs.append(dict(kind=kind, D=D, G=G, fmt=fmt, meta=meta, bits=bits, BH=BH, S=S, dst=dst,
                         cap=cap, pad=pad, mag=mag, recon=recon, seed=seed * 1000 + i))
    return cfgs


def test_sweep_300_configurations():
    cfgs = sweep_configs()
    passed = 0
    for i, c in enumerate(cfgs):
        dtype = torch.bfloat16 if c["fmt"] == "bf16" else torch.float16
        x = synth.kv_tensor(c["BH"], c["S"] + c["pad"], c["D"], keys=c["kind"] == "keys",
                            seed=c["seed"], device="cuda", dtype=torch.float32)
        x = (x * c["mag"]).to(dtype)[:, :c["S"]]      # strided when pad > 0
        what = ("sweep %d/300: %s D=%d G=%d %s meta=%s bits=%d BH=%d S=%d dst=%d cap=%d pad=%d "
                "mag=%g recon=%s" % (i + 1, c["kind"], c["D"], c["G"], c["fmt"], c["meta"], c["bits"],
                                     c["BH"], c["S"], c["dst"], c["cap"], c["pad"], c["mag"],
                                     c["recon"]))
        _run_both(c["kind"], x, c["bits"], c["D"], c["G"], c["meta"], c["cap"], c["dst"], c["recon"],
                  what)
        passed += 1
    note(f"sweep: {passed}/300 configurations bit-exact")
    assert passed == 300
