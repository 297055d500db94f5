"""kivi_decode_attend_noalloc: the decode attend with the library's own
static device array as workspace, for callers that cannot allocate.  Its
output must equal kivi_decode_attend's (same kernels, same plan) bit for bit
and the oracle's within 2e-3, on two calls in a row, the second smaller; a
shape whose partials exceed the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import note, u16
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128


def _case(B, nq, nr, seed):
    Hq, Hkv = 32, 8
    BH = B * Hkv
    cap = ((nq + 31) // 32) * 32
    kx = synth.kv_tensor(BH, nq, keys=True, seed=seed, device="cuda")
    vx = synth.kv_tensor(BH, nq, keys=False, seed=seed, device="cuda")
    kr = synth.residual(BH, nr, keys=True, seed=seed, device="cuda")
    vr = synth.residual(BH, nr, keys=False, seed=seed, device="cuda")
    q = synth.query(B, Hq, seed=seed, device="cuda")
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, 4)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, 4)
    kivi.quantize_keys(kx, ks, 0)
    kivi.quantize_values(vx, vs, 0)
    return dict(B=B, Hq=Hq, Hkv=Hkv, nq=nq, nr=nr, cap=cap, kx=kx, vx=vx, kr=kr, vr=vr, q=q, ks=ks, vs=vs)


def test_noalloc_matches_the_workspace_call_twice():
    for B, nq, nr in ((4, 4096 + 40, 128), (2, 1000, 17)):       # the second call is smaller
        c = _case(B, nq, nr, seed=600 + B)
        note(f"noalloc attend B={B} n_quant={nq} n_res={nr}")
        out_na = kivi.decode_attend_noalloc(c["q"], c["ks"], c["vs"], nq, c["kr"], c["vr"], nr)
        out_ws = kivi.decode_attend(c["q"], c["ks"], c["vs"], nq, c["kr"], c["vr"], nr)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws)
        got = out_na.cpu().numpy().astype(np.float64)
        for b in range(B):
            sl = slice(b * c["Hkv"], (b + 1) * c["Hkv"])
            hk = oracle.Store(oracle.KEYS, c["Hkv"], c["cap"], D, 4)
            hv = oracle.Store(oracle.VALUES, c["Hkv"], c["cap"], D, 4)
            oracle.quantize_keys(u16(c["kx"][sl]), hk, 0, want_recon=False)
            oracle.quantize_values(u16(c["vx"][sl]), hv, 0, want_recon=False)
            ref = oracle.decode_attend(u16(c["q"][b:b + 1]), 1, c["Hq"], c["Hkv"], hk, hv, nq,
                                       u16(c["kr"][sl]), u16(c["vr"][sl]), nr)[0]
            assert float(np.max(np.abs(got[b] - ref))) <= 2e-3


def test_noalloc_refuses_partials_past_the_array():
    """B=32 over 2^24 - 1 store tokens needs about 4 GB of partials: refused
    (KIVI_ERR_WORKSPACE) before anything is launched or looked up."""
    L = kivi.lib()
    fake = 0x10000
    st = kivi.CStore(fake, fake, fake, (1 << 24) * 16, (1 << 24) // 32 * 128, 1 << 24, 4, 32, 128,
                     kivi.KIVI_KEYS, 0)
    sv = kivi.CStore(fake, fake, fake, (1 << 24) * 16, (1 << 24) * 4, 1 << 24, 4, 32, 128,
                     kivi.KIVI_VALUES, 0)
    rc = L.kivi_decode_attend_noalloc(fake, 32, 32, 8, ctypes.byref(st), ctypes.byref(sv), (1 << 24) - 1,
                                      None, None, 0, 0, 0.088, fake, None)
    assert rc == -5
