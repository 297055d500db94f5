"""The largest shapes the ABI admits, where the kernels' 32-bit offset
arguments are tightest: one slab of n_quant = 2^24 - 1 store tokens (the
attend's token bound; the last key group is ragged) plus a residual window.

  * the flushes are compared with the oracle over the whole slab, in token
    windows of 2^18 (key windows start on a group, so each window is an
    independent flush; the oracle runs the windows on a thread pool), the
    last window ending in the ragged group;
  * the dequantize is compared with the oracle on the same windows;
  * the attend (uniform and variable-length) must equal dense attention in
    float64 over the library's own dequantization of the same store (a
    property that holds at any size: the fused kernel reads the packed
    store, the reference reads dequantize's fp16 rows), within 2e-3.
About 50 GB of device memory."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import note, u16
from oracle_pool import pmap, threads
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128
N = (1 << 24) - 1
CAP = 1 << 24


def test_largest_single_slab():
    B, Hq, Hkv, nr = 1, 8, 1, 100
    note(f"limits: one slab of {N} store tokens, {nr} residual")
    kx = synth.kv_tensor(1, N, keys=True, seed=77, device="cuda")
    vx = synth.kv_tensor(1, N, keys=False, seed=78, device="cuda")
    ks = kivi.Store(kivi.KIVI_KEYS, 1, CAP, 4)
    vs = kivi.Store(kivi.KIVI_VALUES, 1, CAP, 4)
    kivi.quantize_keys(kx, ks, 0)
    kivi.quantize_values(vx, vs, 0)
    torch.cuda.synchronize()

    # the whole slab against the oracle, window by window
    W = 1 << 18
    windows = [(t0, min(W, N - t0)) for t0 in range(0, N, W)]
    for kind, x, st in ((oracle.KEYS, kx, ks), (oracle.VALUES, vx, vs)):
        fn = oracle.quantize_keys if kind == oracle.KEYS else oracle.quantize_values
        for i in range(0, len(windows), threads()):
            part = windows[i:i + threads()]
            note(f"limits: oracle {'keys' if kind == oracle.KEYS else 'values'} tokens "
                 f"[{part[0][0]}, {part[-1][0] + part[-1][1]})")
            host = []
            for t0, n in part:
                g0, g1 = (t0 // 32, (t0 + n + 31) // 32) if kind == oracle.KEYS else (t0, t0 + n)
                host.append((t0, n, u16(x[:, t0:t0 + n]),
                             st.codes[:, t0:t0 + n].cpu().numpy().view(np.uint32),
                             st.scale[:, g0:g1].cpu().numpy().view(np.uint32),
                             st.zero[:, g0:g1].cpu().numpy().view(np.uint32),
                             u16(kivi.dequantize(st, t0, n))))

            def one(h):
                t0, n, xh, codes, scale, zero, rec = h
                hs = oracle.Store(kind, 1, n + (-n) % 32, D, 4, 32)
                hrec = fn(xh, hs, 0, want_recon=True)
                m = scale.shape[1]
                return (t0, np.array_equal(codes, hs.codes[:, :n]),
                        np.array_equal(scale, hs.scale[:, :m].view(np.uint32)),
                        np.array_equal(zero, hs.zero[:, :m].view(np.uint32)),
                        np.array_equal(rec, hrec))
            for t0, *ok in pmap(one, host):
                assert all(ok), f"window at token {t0}: codes/scale/zero/dequantize equal {ok}"
            del host
    del kx, vx
    torch.cuda.empty_cache()

    kr = synth.residual(1, nr, keys=True, seed=79, device="cuda")
    vr = synth.residual(1, nr, keys=False, seed=79, device="cuda")
    q = synth.query(B, Hq, seed=79, device="cuda")
    out = kivi.decode_attend(q, ks, vs, N, kr, vr, nr)
    nq_t = torch.full((1,), N, dtype=torch.int32, device="cuda")
    nr_t = torch.full((1,), nr, dtype=torch.int32, device="cuda")
    out_v = kivi.decode_attend_varlen(q, ks, vs, nq_t, N, kr, vr, nr_t, nr)
    torch.cuda.synchronize()

    # dense float64 attention over dequantize's rows and the residual
    kh = torch.cat([kivi.dequantize(ks, 0, N)[0], kr[0, :nr]]).double()
    scores = (kh @ q[0].double().T) / np.sqrt(D)          # [N + nr][Hq]
    del kh
    p = torch.softmax(scores, dim=0)
    del scores
    vh = torch.cat([kivi.dequantize(vs, 0, N)[0], vr[0, :nr]]).double()
    ref = (p.T @ vh).cpu().numpy()                         # [Hq][D]
    del vh, p
    for got in (out, out_v):
        err = float(np.max(np.abs(got[0].cpu().numpy().astype(np.float64) - ref)))
        assert err <= 2e-3, f"max-abs error {err:.3e}"
