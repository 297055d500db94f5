"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph on
ROCm): a key flush, a value flush, a dequantize and an attend are captured
once and replayed several times, with the program's own eager work and
synchronizations between replays, and every replay is compared with the
eager result.  None of the calls records a memset or allocates, so a replay
must reproduce the eager outputs exactly (the attend to the bit as well:
same kernels, same launch shapes)."""
import numpy as np
import pytest
import torch

from gpu_util import note, u16
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("bits", [4, 2])
def test_graph_replays_match_eager(bits):
    B, Hq, Hkv, nq, nr = 2, 32, 8, 1000, 37
    BH = B * Hkv
    kx = synth.kv_tensor(BH, nq, keys=True, seed=4242, device="cuda")
    vx = synth.kv_tensor(BH, nq, keys=False, seed=4242, device="cuda")
    kr = synth.residual(BH, nr, keys=True, seed=4242, device="cuda")
    vr = synth.residual(BH, nr, keys=False, seed=4242, device="cuda")
    q = synth.query(B, Hq, seed=4242, device="cuda")
    cap = 1024
    ks = kivi.Store(kivi.KIVI_KEYS, BH, cap, bits)
    vs = kivi.Store(kivi.KIVI_VALUES, BH, cap, bits)
    recon = torch.empty((BH, nq, 128), dtype=torch.float16, device="cuda")
    deq = torch.empty_like(recon)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    ws = kivi.attend_workspace(kivi.attend_workspace_bytes(B, Hq, Hkv, nq, nr))

    def work(stream):
        kivi.quantize_keys(kx, ks, 0, recon, stream=stream)
        kivi.quantize_values(vx, vs, 0, stream=stream)
        kivi.dequantize(vs, 0, nq, out=deq, stream=stream)
        kivi.decode_attend(q, ks, vs, nq, kr, vr, nr, out=out, workspace=ws, stream=stream)

    note(f"graph capture and replay bits={bits}")
    work(None)
    torch.cuda.synchronize()
    # the windows the calls write: tokens [0, nq) of the codes and of the
    # per-token value metadata, every key group row (32 x 32 >= nq)
    def outputs():
        return (ks.codes[:, :nq], ks.scale, vs.codes[:, :nq], vs.scale[:, :nq], recon, deq, out)
    want = tuple(t.clone() for t in outputs())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work(s)                                   # warm the stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            work(s)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays that overwrites every output
        for t in (ks.codes, vs.codes):
            t.fill_(0x5A5A5A5A)
        for t in (ks.scale, vs.scale, out):
            t.fill_(-3.5)
        recon.fill_(7.0)
        deq.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, a, b in zip(("key codes", "key scale", "value codes", "value scale", "recon",
                               "dequantize", "attend"), got, want):
            assert torch.equal(a.view(torch.int8) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.int8) if b.dtype != torch.float32 else b.view(torch.int32)), \
                f"replay {rep}: {name} differs from the eager result"
    # the eager call still works after the graph
    work(None)
    torch.cuda.synchronize()
    assert np.array_equal(u16(recon), u16(want[4]))
