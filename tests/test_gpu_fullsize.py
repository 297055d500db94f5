"""GPU parity at full workload sizes, in the launch configurations the
benchmark times.

* Long-context full-cache flush: 36 layers x B=1 x H_kv=8 folded into
  BH=288 slabs of S=32768 tokens, one launch per tensor, bits 4 and 2.  The
  oracle recomputes sampled slabs; every element is checked against a
  property that holds at any size (the reconstruction error bound, and the
  dequantize kernel reproducing the fused reconstruction).
* Decode-time incremental flush: B=32 sequences x 36 layers x H_kv=8, 128
  new tokens per slab flushed at token 4096 of an existing 4-bit store; per
  layer (72 launches) and layer-folded (2 launches) must agree, the 4096
  older tokens must be untouched, and sampled slabs match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (CODE_SENTINEL, META_SENTINEL, assert_store_equal, assert_u16_equal,
                      device_store, host_store, note, u16)
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128
LAYERS, HKV = 36, 8


def _slice_store(st: kivi.Store, a: int, b: int) -> kivi.Store:
    return kivi.Store(st.kind, b - a, st.cap, st.bits, codes=st.codes[a:b], scale=st.scale[a:b],
                      zero=st.zero[a:b])


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
def test_full_cache_flush(kind, bits):
    BH, S = LAYERS * HKV, 32768
    k = kivi.KIVI_KEYS if kind == "keys" else kivi.KIVI_VALUES
    note(f"full-cache {kind} bits={bits}: generating {BH}x{S}x{D}")
    x = synth.kv_tensor(BH, S, keys=(kind == "keys"), seed=1003, device="cuda")
    st = kivi.Store(k, BH, S, bits)
    note(f"full-cache {kind} bits={bits}: flush")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, 0)
    torch.cuda.synchronize()

    # sampled slabs against the oracle
    for bh in (0, 137, BH - 1):
        note(f"full-cache {kind} bits={bits}: oracle slab {bh}")
        hs = oracle.Store(oracle.KEYS if kind == "keys" else oracle.VALUES, 1, S, D, bits)
        fn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
        fn(u16(x[bh:bh + 1]), hs, 0, want_recon=False)
        assert_store_equal(_slice_store(st, bh, bh + 1), hs, what=f"{kind} slab {bh}")

    # every element: dequantize, then |x - recon| <= scale/2 + rounding slack,
    # and the fused reconstruction equals the dequantize kernel's output
    L = (1 << bits) - 1
    chunk = 16
    for b0 in range(0, BH, chunk):
        b1 = min(BH, b0 + chunk)
        sub = _slice_store(st, b0, b1)
        rec = kivi.dequantize(sub, 0, S)
        xf = x[b0:b1].float()
        rf = rec.float()
        if kind == "keys":
            sc = st.scale[b0:b1].repeat_interleave(32, dim=1)
            ze = st.zero[b0:b1].repeat_interleave(32, dim=1)
        else:
            sc = st.scale[b0:b1].repeat_interleave(32, dim=2)
            ze = st.zero[b0:b1].repeat_interleave(32, dim=2)
        ulp16 = torch.where(rf.abs() < 2.0 ** -14, torch.full_like(rf, 2.0 ** -24),
                            torch.exp2(torch.floor(torch.log2(rf.abs().clamp_min(2.0 ** -14)))) * 2.0 ** -10)
        bound = sc / 2 + 0.5 * ulp16 + 2.0 ** -22 * (ze.abs() + L * sc)
        assert bool(((xf - rf).abs() <= bound).all()), f"error bound violated in slabs {b0}..{b1}"
        if b0 == 0:
            fused = torch.empty_like(x[b0:b1])
            st2 = kivi.Store(k, b1 - b0, S, bits)
            (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x[b0:b1], st2, 0, fused)
            assert torch.equal(fused.view(torch.int16), rec.view(torch.int16))
            assert torch.equal(st2.codes, sub.codes)
        del rec, xf, rf, sc, ze, ulp16, bound
    torch.cuda.synchronize()


def test_decode_incremental_flush():
    B, T0, NEW, bits = 32, 4096, 128, 4
    BH = LAYERS * B * HKV                       # layer-major: slab = (l*B + b)*HKV + kv
    cap = T0 + NEW
    note("decode flush: building stores")
    xk = synth.residual(BH, NEW, keys=True, seed=1004, device="cuda")
    xv = synth.residual(BH, NEW, keys=False, seed=1004, device="cuda")
    stores = {}
    for name, kind in (("k", kivi.KIVI_KEYS), ("v", kivi.KIVI_VALUES)):
        for mode in ("folded", "per_layer"):
            stores[name, mode] = device_store(kind, BH, cap, bits)
    # the existing 4096 tokens: a fixed byte pattern that must survive
    g = torch.Generator(device="cuda").manual_seed(9)
    for (name, mode), st in stores.items():
        st.codes[:, :T0].copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, st.codes[:, :T0].shape,
                                             generator=g, device="cuda", dtype=torch.int32))
    old_codes = stores["k", "folded"].codes[:, :T0].clone()

    note("decode flush: layer-folded (2 launches)")
    kivi.quantize_keys(xk, stores["k", "folded"], T0)
    kivi.quantize_values(xv, stores["v", "folded"], T0)
    note("decode flush: per layer (72 launches)")
    per = B * HKV
    for l in range(LAYERS):
        a, b = l * per, (l + 1) * per
        kivi.quantize_keys(xk[a:b], _slice_store(stores["k", "per_layer"], a, b), T0)
        kivi.quantize_values(xv[a:b], _slice_store(stores["v", "per_layer"], a, b), T0)
    torch.cuda.synchronize()

    for name in ("k", "v"):
        f, p = stores[name, "folded"], stores[name, "per_layer"]
        assert torch.equal(f.codes[:, T0:], p.codes[:, T0:])
        assert torch.equal(f.scale.view(torch.int32), p.scale.view(torch.int32))
        assert torch.equal(f.zero.view(torch.int32), p.zero.view(torch.int32))
    assert torch.equal(stores["k", "folded"].codes[:, :T0], old_codes)
    # metadata outside the new window is untouched
    assert bool((stores["k", "folded"].scale[:, :T0 // 32] == META_SENTINEL).all())
    assert bool((stores["v", "folded"].scale[:, :T0] == META_SENTINEL).all())

    for bh in (0, 1111, BH - 1):
        note(f"decode flush: oracle slab {bh}")
        for name, kind, x in (("k", oracle.KEYS, xk), ("v", oracle.VALUES, xv)):
            hs = oracle.Store(kind, 1, cap, D, bits)
            (oracle.quantize_keys if name == "k" else oracle.quantize_values)(
                u16(x[bh:bh + 1]), hs, T0, want_recon=False)
            got = _slice_store(stores[name, "folded"], bh, bh + 1)
            codes = got.codes.cpu().numpy().view(np.uint32)
            assert np.array_equal(codes[:, T0:], hs.codes[:, T0:])
            g0 = T0 // 32 if name == "k" else T0
            assert np.array_equal(got.scale.cpu().numpy()[:, g0:].view(np.uint32),
                                  hs.scale[:, g0:].view(np.uint32))
            assert np.array_equal(got.zero.cpu().numpy()[:, g0:].view(np.uint32),
                                  hs.zero[:, g0:].view(np.uint32))
