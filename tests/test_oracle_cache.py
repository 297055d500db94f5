"""Pins for the oracle's model of the decode-loop cache (oracle.CacheModel).

  * the flushed-token counts reproduce the flush/layer column of the Metal
    post's end-to-end record (559 -> 512, 2059 -> 2016, 8209 -> 8160 tokens
    with residual length = group size = 32), and between prompt and steps the
    fp16 tail always holds between R and R + F - 1 tokens;
  * stores built by many small flushes equal one flush of the same prefix
    (every group depends only on its own tokens);
  * each step's attention is torch's float64 SDPA over [dequantized store
    tokens ; every later fp16 token including the step's own].
"""
import numpy as np
import pytest
import torch

D = 128


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def _w(u):
    return u.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("S,Q", [(559, 512), (2059, 2016), (8209, 8160)])
def test_prompt_flush_matches_the_generation_record(orc, S, Q):
    rng = np.random.default_rng(S)
    m = orc.CacheModel(1, 1, 1, capacity=8192, R=32, F=32)
    m.prefill(_f16(rng.standard_normal((1, S, D))), _f16(rng.standard_normal((1, S, D))))
    assert m.n_quant == Q


@pytest.mark.parametrize("R,F", [(64, 32), (128, 128), (0, 32)])
def test_incremental_stores_equal_one_flush_and_tail_stays_in_window(orc, R, F):
    rng = np.random.default_rng(R + F)
    layers, batch, kvh, Hq = 2, 1, 2, 4
    slabs = layers * batch * kvh
    m = orc.CacheModel(layers, batch, kvh, capacity=512, R=R, F=F)
    S0 = 100
    m.prefill(_f16(rng.standard_normal((slabs, S0, D)) * 3), _f16(rng.standard_normal((slabs, S0, D))))
    flushes = 0
    for step in range(300):
        before = m.n_quant
        m.step(_f16(rng.standard_normal((slabs, D)) * 3), _f16(rng.standard_normal((slabs, D))),
               _f16(rng.standard_normal((layers, batch, Hq, D))), Hq)
        flushes += m.n_quant != before
        tail = m.length - m.n_quant
        if m.length >= R:
            assert R <= tail <= R + F - 1, (step, tail)
        assert m.n_quant % F == 0
    assert flushes >= 2
    Q = m.n_quant
    ks = orc.Store(orc.KEYS, slabs, 512, D, 4)
    vs = orc.Store(orc.VALUES, slabs, 512, D, 4)
    orc.quantize_keys(np.ascontiguousarray(m.k[:, :Q]), ks, 0, want_recon=False)
    orc.quantize_values(np.ascontiguousarray(m.v[:, :Q]), vs, 0, want_recon=False)
    assert np.array_equal(ks.codes, m.kstore.codes) and np.array_equal(vs.codes, m.vstore.codes)
    assert np.array_equal(ks.scale.view(np.uint32), m.kstore.scale.view(np.uint32))
    assert np.array_equal(ks.zero.view(np.uint32), m.kstore.zero.view(np.uint32))
    assert np.array_equal(vs.scale.view(np.uint32), m.vstore.scale.view(np.uint32))
    assert np.array_equal(vs.zero.view(np.uint32), m.vstore.zero.view(np.uint32))


def test_step_attention_is_sdpa_over_store_then_fp16_tail(orc):
    rng = np.random.default_rng(5)
    layers, batch, kvh, Hq, R, F = 2, 2, 1, 2, 32, 32
    slabs = layers * batch * kvh
    m = orc.CacheModel(layers, batch, kvh, capacity=256, R=R, F=F)
    m.prefill(_f16(rng.standard_normal((slabs, 90, D))), _f16(rng.standard_normal((slabs, 90, D))))
    for _ in range(7):                       # cross one flush (at length 96)
        kn, vn = _f16(rng.standard_normal((slabs, D))), _f16(rng.standard_normal((slabs, D)))
        q = _f16(rng.standard_normal((layers, batch, Hq, D)))
        nq = m.n_quant
        kd = _w(orc.dequantize(m.kstore, 0, nq)) if nq else np.zeros((slabs, 0, D))
        vd = _w(orc.dequantize(m.vstore, 0, nq)) if nq else np.zeros((slabs, 0, D))
        got = m.step(kn, vn, q, Hq)
        for layer in range(layers):
            for b in range(batch):
                s = layer * batch + b
                kk = np.concatenate([kd[s], _w(m.k[s, nq:])], axis=0)
                vv = np.concatenate([vd[s], _w(m.v[s, nq:])], axis=0)
                qt = torch.from_numpy(_w(q[layer, b])).reshape(1, Hq, 1, D)
                kt = torch.from_numpy(kk).reshape(1, 1, -1, D).expand(1, Hq, -1, D)
                vt = torch.from_numpy(vv).reshape(1, 1, -1, D).expand(1, Hq, -1, D)
                want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, D).numpy()
                assert np.max(np.abs(got[layer, b] - want)) < 1e-12
    assert m.n_quant == 64                    # flush_count(97, 32, 32)


def test_chunked_prompt_matches_the_whole_prompt_and_the_2048_chunking(orc):
    """An 8209-token prompt fed in 2048-token chunks (the pages' runtime
    chunks prefill at 2048: [Metal post] "Four benchmarks that lied", Lie #1)
    flushes 8160 tokens per layer (the Generation 1 flush/layer column with
    R = G = 32) and builds the same stores as the whole prompt at once; so do
    ragged chunk lengths that are not multiples of the group size, with
    decode steps in between."""
    rng = np.random.default_rng(8209)
    S, slabs = 8209, 2
    k = _f16(rng.standard_normal((slabs, S, D)) * 3)
    v = _f16(rng.standard_normal((slabs, S, D)))
    whole = orc.CacheModel(1, 1, slabs, capacity=8192, R=32, F=32)
    whole.prefill(k, v)
    chunked = orc.CacheModel(1, 1, slabs, capacity=8192, R=32, F=32)
    counts = []
    for c0 in range(0, S, 2048):
        chunked.prefill(k[:, c0:c0 + 2048], v[:, c0:c0 + 2048])
        counts.append(chunked.n_quant)
    assert counts == [orc.flush_count(min(S, c0 + 2048), 32, 32) for c0 in range(0, S, 2048)]
    assert chunked.n_quant == whole.n_quant == 8160
    for a, b in ((chunked.kstore, whole.kstore), (chunked.vstore, whole.vstore)):
        assert np.array_equal(a.codes, b.codes)
        assert np.array_equal(a.scale.view(np.uint32), b.scale.view(np.uint32))
        assert np.array_equal(a.zero.view(np.uint32), b.zero.view(np.uint32))
    # ragged chunks with steps between them, R = 64, F = 32
    m = orc.CacheModel(1, 1, slabs, capacity=1024, R=64, F=32)
    ref = orc.CacheModel(1, 1, slabs, capacity=1024, R=64, F=32)
    pos = 0
    for n in (45, 1, 100, 77, 31, 200):
        m.prefill(k[:, pos:pos + n], v[:, pos:pos + n])
        pos += n
        m.step(k[:, pos], v[:, pos], _f16(rng.standard_normal((1, 1, 4, D))), 4)
        pos += 1
        assert m.n_quant == orc.flush_count(pos, 64, 32)
    ref.prefill(k[:, :pos], v[:, :pos])
    assert m.n_quant == ref.n_quant
    assert np.array_equal(m.kstore.codes, ref.kstore.codes)
    assert np.array_equal(m.vstore.codes, ref.vstore.codes)
