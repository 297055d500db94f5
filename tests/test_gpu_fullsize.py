"""GPU parity at full workload sizes, element by element, in the launch
configurations the benchmark times.

* Long-context full-cache flush: 36 layers x B=1 x H_kv=8 folded into
  BH=288 slabs of S=32768 tokens, one launch per tensor, keys and values,
  bits 4 and 2.  Every slab's codes, scales and zeros, and the dequantized
  fp16 output of the whole cache, are compared with the oracle's bit for bit
  (the oracle runs one slab per task on a thread pool).
* Decode-time incremental flush: B=32 sequences x 36 layers x H_kv=8, 128
  new tokens per slab flushed at token 4096 of an existing 4-bit store; per
  layer (72 launches) and layer-folded (2 launches) must agree, the 4096
  older tokens must be untouched, and all 9216 slabs match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import META_SENTINEL, note, u16
from oracle_pool import pmap, threads
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128
LAYERS, HKV = 36, 8


def _slice_store(st: kivi.Store, a: int, b: int) -> kivi.Store:
    return kivi.Store(st.kind, b - a, st.cap, st.bits, codes=st.codes[a:b], scale=st.scale[a:b],
                      zero=st.zero[a:b])


def _first_diff(a, b):
    bad = np.argwhere(a != b)
    return f"{len(bad)} differ, first at {bad[0].tolist()}" if len(bad) else "equal"


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("kind", ["keys", "values"])
def test_full_cache_flush(kind, bits):
    BH, S = LAYERS * HKV, 32768
    k = kivi.KIVI_KEYS if kind == "keys" else kivi.KIVI_VALUES
    okind = oracle.KEYS if kind == "keys" else oracle.VALUES
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    note(f"full-cache {kind} bits={bits}: generating {BH}x{S}x{D}")
    x = synth.kv_tensor(BH, S, keys=(kind == "keys"), seed=1003, device="cuda")
    st = kivi.Store(k, BH, S, bits)
    note(f"full-cache {kind} bits={bits}: flush (one launch)")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, 0)
    torch.cuda.synchronize()

    # every slab against the oracle, in chunks of slabs: codes, scale, zero
    # and the dequantize kernel's fp16 output
    chunk = 4 * threads()
    for b0 in range(0, BH, chunk):
        b1 = min(BH, b0 + chunk)
        note(f"full-cache {kind} bits={bits}: oracle slabs {b0}..{b1 - 1} on {threads()} threads")
        xh = u16(x[b0:b1])
        codes = st.codes[b0:b1].cpu().numpy().view(np.uint32)
        scale = st.scale[b0:b1].cpu().numpy().view(np.uint32)
        zero = st.zero[b0:b1].cpu().numpy().view(np.uint32)
        rec = u16(kivi.dequantize(_slice_store(st, b0, b1), 0, S))

        def one(i):
            hs = oracle.Store(okind, 1, S, D, bits)
            hrec = ofn(xh[i:i + 1], hs, 0, want_recon=True)
            return (np.array_equal(codes[i], hs.codes[0]),
                    np.array_equal(scale[i], hs.scale[0].view(np.uint32)),
                    np.array_equal(zero[i], hs.zero[0].view(np.uint32)),
                    np.array_equal(rec[i], hrec[0]))
        res = pmap(one, range(b1 - b0))
        bad = [(b0 + i, r) for i, r in enumerate(res) if not all(r)]
        if bad:
            bh = bad[0][0]
            hs = oracle.Store(okind, 1, S, D, bits)
            hrec = ofn(xh[bh - b0:bh - b0 + 1], hs, 0, want_recon=True)
            raise AssertionError(
                f"{kind} bits={bits}: {len(bad)} slabs differ from the oracle, first slab {bh} "
                f"(codes/scale/zero/dequantize equal: {bad[0][1]}); codes "
                f"{_first_diff(codes[bh - b0], hs.codes[0])}; dequantize "
                f"{_first_diff(rec[bh - b0], hrec[0])}")
        del xh, codes, scale, zero, rec

    # the fused reconstruction of the flush equals the dequantize kernel's
    # output (checked on the first 16 slabs)
    sub = _slice_store(st, 0, 16)
    fused = torch.empty_like(x[:16])
    st2 = kivi.Store(k, 16, S, bits)
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x[:16], st2, 0, fused)
    rec = kivi.dequantize(sub, 0, S)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), rec.view(torch.int16))
    assert torch.equal(st2.codes, sub.codes)


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
            st = kivi.Store(kind, BH, cap, bits)
            st.scale.fill_(META_SENTINEL)
            st.zero.fill_(META_SENTINEL)
            stores[name, mode] = st
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

    # every slab's new window against the oracle (flushed at the same offset)
    per_task = 32
    for name, okind, x, ofn in (("k", oracle.KEYS, xk, oracle.quantize_keys),
                                ("v", oracle.VALUES, xv, oracle.quantize_values)):
        note(f"decode flush: oracle, all {BH} slabs of {name} on {threads()} threads")
        st = stores[name, "folded"]
        g0 = T0 // 32 if name == "k" else T0
        xh = u16(x)
        codes = st.codes[:, T0:].cpu().numpy().view(np.uint32)
        scale = st.scale[:, g0:].cpu().numpy().view(np.uint32)
        zero = st.zero[:, g0:].cpu().numpy().view(np.uint32)

        def one(a):
            b = min(BH, a + per_task)
            hs = oracle.Store(okind, b - a, cap, D, bits)
            ofn(xh[a:b], hs, T0, want_recon=False)
            return (np.array_equal(codes[a:b], hs.codes[:, T0:]),
                    np.array_equal(scale[a:b], hs.scale[:, g0:].view(np.uint32)),
                    np.array_equal(zero[a:b], hs.zero[:, g0:].view(np.uint32)))
        res = pmap(one, range(0, BH, per_task))
        bad = [i * per_task for i, r in enumerate(res) if not all(r)]
        assert not bad, f"{name}: slabs from {bad[:5]} differ from the oracle"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["keys", "values"])
@pytest.mark.parametrize("Dh", [80, 96, 144, 160])
def test_other_head_dims_at_full_size(Dh, kind, fmt):
    """The head_dims whose rows are packed (fp16 key rows of head_dim/8
    lanes, value rows of whole DPP quads) at the element count of the full
    cache: 288 * 128 / head_dim slabs of 32768 tokens in one launch, as the
    benchmark's head_dim rows time them.  Six slabs (both ends and the
    middle) are compared whole with the oracle: codes, scale, zero, and the
    dequantize kernel's output."""
    S, bits = 32768, 4
    BH = LAYERS * HKV * D // Dh
    k = kivi.KIVI_KEYS if kind == "keys" else kivi.KIVI_VALUES
    okind = oracle.KEYS if kind == "keys" else oracle.VALUES
    ofn = oracle.quantize_keys if kind == "keys" else oracle.quantize_values
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    note(f"full-size head_dim {Dh} {fmt} {kind}: generating {BH}x{S}x{Dh}")
    x = synth.kv_tensor(BH, S, Dh, keys=(kind == "keys"), seed=1009, device="cuda", dtype=dtype)
    st = kivi.Store(k, BH, S, bits, head_dim=Dh)
    note(f"full-size head_dim {Dh} {fmt} {kind}: flush (one launch)")
    (kivi.quantize_keys if kind == "keys" else kivi.quantize_values)(x, st, 0)
    torch.cuda.synchronize()
    sample = [0, 1, BH // 3, BH // 2, BH - 2, BH - 1]
    idx = torch.tensor(sample, device="cuda")
    sub = kivi.Store(k, len(sample), S, bits, head_dim=Dh, codes=st.codes[idx], scale=st.scale[idx],
                     zero=st.zero[idx])
    rec = u16(kivi.dequantize(sub, 0, S, dtype=dtype))
    xh = u16(x[idx])
    codes = sub.codes.cpu().numpy().view(np.uint32)
    scale = sub.scale.cpu().numpy().view(np.uint32)
    zero = sub.zero.cpu().numpy().view(np.uint32)
    del x, st
    note(f"full-size head_dim {Dh} {fmt} {kind}: oracle over slabs {sample}")

    def one(i):
        hs = oracle.Store(okind, 1, S, Dh, bits)
        hrec = ofn(xh[i:i + 1], hs, 0, want_recon=True, fmt=fmt)
        return (_first_diff(codes[i], hs.codes[0]), _first_diff(scale[i], hs.scale[0].view(np.uint32)),
                _first_diff(zero[i], hs.zero[0].view(np.uint32)), _first_diff(rec[i], hrec[0]))
    for bh, r in zip(sample, pmap(one, range(len(sample)))):
        assert r == ("equal",) * 4, f"D={Dh} {fmt} {kind} slab {bh}: codes/scale/zero/dequantize {r}"
