"""GPU parity of the decode-loop cache (include/kivi_cache.h) against the
oracle's CacheModel, step by step: every layer's attention output of every
step within 2e-3 max-abs, the flush launches where the rule puts them, and
at the end the stores bit-exact and the fp16 ring contents (read in logical
order from the ring's head) byte-identical to the model's fp16 tail."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import note, u16
from kv_cache_quantization_quantize_amd import kivi, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D = 128
TOL = 2e-3

CASES = [
    # layers, batch, kv_heads, Hq, bits, R, F, capacity, prompt, steps, scale/zero format
    (2, 2, 2, 8, 4, 64, 32, 512, 150, 100, "f32"),       # F = G
    (1, 2, 8, 32, 4, 128, 128, 512, 200, 200, "f32"),    # 128-token flushes (F = R)
    (2, 1, 2, 4, 2, 0, 32, 256, 31, 70, "f32"),          # no fp16 window kept (R = 0), 2-bit
    (3, 1, 1, 8, 4, 64, 32, 256, 10, 120, "f32"),        # prompt shorter than R
    (1, 3, 2, 16, 4, 32, 32, 256, 0, 90, "f32"),         # empty prompt
    (2, 2, 2, 8, 4, 64, 32, 512, 150, 100, "f16"),       # binary16 scale/zero
    (2, 1, 2, 4, 2, 0, 32, 256, 31, 70, "f16"),
    (2, 2, 2, 8, 4, 64, 32, 512, 150, 100, "bf16"),      # a bfloat16 cache
    (1, 2, 8, 32, 2, 128, 128, 512, 200, 140, "bf16"),
]


def _meta_equal(gpu: torch.Tensor, host: np.ndarray) -> bool:
    """Metadata equal as bit patterns (binary16 stores: the host holds the
    binary16 values widened, so their conversion is exact)."""
    g = gpu.cpu().numpy()
    if g.dtype == np.float16:
        return np.array_equal(g.view(np.uint16), oracle.f32_to_f16(host))
    return np.array_equal(g.view(np.uint32), np.ascontiguousarray(host).view(np.uint32))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%d-B%d-H%d-q%d-b%d-R%d-F%d-S%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[8], c[10]))
def test_decode_loop_matches_model(case):
    """The last field is the scale/zero format ("f32", "f16") or "bf16" for a
    bfloat16 cache (binary32 scale/zero; the same 2e-3 tolerance)."""
    _decode_loop(case, 32)


@pytest.mark.parametrize("G,case", [
    (64, (2, 2, 2, 8, 4, 128, 64, 512, 150, 140, "f32")),
    (128, (1, 2, 8, 32, 4, 128, 128, 512, 200, 200, "f16")),
    (64, (2, 1, 2, 8, 2, 64, 64, 256, 70, 90, "bf16")),
], ids=["G64", "G128-meta16", "G64-bf16"])
def test_decode_loop_group_sizes(G, case):
    """Caches with groups of 64 and 128 (flush units multiples of the group)."""
    _decode_loop(case, G)


@pytest.mark.parametrize("Dh,case", [
    (64, (2, 2, 2, 8, 4, 64, 32, 256, 100, 90, "f32")),
    (96, (1, 2, 2, 8, 2, 64, 32, 256, 70, 80, "bf16")),
    (256, (1, 1, 2, 8, 4, 32, 32, 256, 40, 70, "f32")),
], ids=["D64", "D96-bf16", "D256"])
def test_decode_loop_head_dims(Dh, case):
    """Caches at other head_dims (the attend at 64 and 256 on their own MFMA
    geometry, at 96 padded onto the 128-channel one)."""
    _decode_loop(case, 32, Dh)


def _decode_loop(case, G, Dh=D):
    layers, batch, kvh, Hq, bits, R, F, cap, S0, steps, variant = case
    sched = ([("chunk", S0)] if S0 else []) + [("steps", steps)]
    _run_schedule(layers, batch, kvh, Hq, bits, R, F, cap, variant, sched, G, Dh, seed=9000 + S0 + R)
    print(f"{case}: ok")


def _run_schedule(layers, batch, kvh, Hq, bits, R, F, cap, variant, schedule, G=32, Dh=D, seed=0):
    """Drive the GPU cache and the oracle's CacheModel through the same
    schedule of ("chunk", n) prompt chunks and ("steps", n) decode steps:
    token counts equal after every event, every step's attention within
    TOL, and at the end the stores bit-exact and the rings' fp16 tokens (in
    logical order from the head) byte-identical to the model's tail."""
    bf16 = variant == "bf16"
    meta = "f32" if bf16 else variant
    dtype = torch.bfloat16 if bf16 else torch.float16
    fmt = "bf16" if bf16 else "f16"
    slabs = layers * batch * kvh
    per = batch * kvh
    note(f"cache layers={layers} batch={batch} kv_heads={kvh} Hq={Hq} bits={bits} R={R} F={F} "
         f"capacity={cap} G={G} D={Dh} {variant} schedule={schedule}")
    c = kivi.Cache(layers, batch, kvh, cap, bits, R, F, meta=meta, dtype=dtype, group=G, head_dim=Dh)
    m = oracle.CacheModel(layers, batch, kvh, cap, bits, R, F, D=Dh, meta=meta, fmt=fmt, G=G)
    ws = kivi.attend_workspace(c.attend_workspace_bytes(Hq))
    worst = 0.0
    step = 0
    for e, (what, n) in enumerate(schedule):
        if what == "chunk":
            k0 = synth.kv_tensor(slabs, n, Dh, keys=True, seed=seed + 17 * e, device="cuda", dtype=dtype)
            v0 = synth.kv_tensor(slabs, n, Dh, keys=False, seed=seed + 17 * e, device="cuda", dtype=dtype)
            c.prefill(k0, v0)
            m.prefill(u16(k0), u16(v0))
            assert (c.length, c.n_quant) == (m.length, m.n_quant), (e, what, n)
            continue
        for _ in range(n):
            kn = synth.kv_tensor(slabs, 1, Dh, keys=True, seed=seed * 1000 + step, device="cuda",
                                 dtype=dtype)[:, 0].contiguous()
            vn = synth.kv_tensor(slabs, 1, Dh, keys=False, seed=seed * 1000 + step, device="cuda",
                                 dtype=dtype)[:, 0].contiguous()
            q = synth.query(layers * batch, Hq, Dh, seed=seed * 1000 + step, device="cuda").to(dtype) \
                .view(layers, batch, Hq, Dh)
            outs = []
            for layer in range(layers):
                c.append(layer, kn[layer * per:(layer + 1) * per], vn[layer * per:(layer + 1) * per])
                outs.append(c.attend(layer, q[layer].contiguous(), workspace=ws))
            before = c.n_quant
            launches = c.end_step()
            torch.cuda.synchronize()
            ref = m.step(u16(kn), u16(vn), u16(q), Hq)
            assert (c.length, c.n_quant) == (m.length, m.n_quant), step
            assert launches == (2 if c.n_quant != before else 0)
            for layer in range(layers):
                err = float(np.max(np.abs(outs[layer].cpu().numpy().astype(np.float64) - ref[layer])))
                worst = max(worst, err)
                assert err <= TOL, f"step {step} layer {layer}: max-abs error {err:.3e}"
            step += 1
    Q = c.n_quant
    ks, vs = c.stores()
    torch.cuda.synchronize()
    g = Q // G
    assert np.array_equal(ks.codes[:, :Q].cpu().numpy().view(np.uint32), m.kstore.codes[:, :Q])
    assert np.array_equal(vs.codes[:, :Q].cpu().numpy().view(np.uint32), m.vstore.codes[:, :Q])
    assert _meta_equal(ks.scale[:, :g], m.kstore.scale[:, :g])
    assert _meta_equal(ks.zero[:, :g], m.kstore.zero[:, :g])
    assert _meta_equal(vs.scale[:, :Q], m.vstore.scale[:, :Q])
    assert _meta_equal(vs.zero[:, :Q], m.vstore.zero[:, :Q])
    kr, vr = c.rings()
    rows = [(c.head + i) % c.ring for i in range(c.n_res)]
    assert c.n_res == m.length - Q
    assert np.array_equal(u16(kr[:, rows]), m.k[:, Q:])
    assert np.array_equal(u16(vr[:, rows]), m.v[:, Q:])
    return worst


CHUNKED = [
    # layers, batch, kv_heads, Hq, bits, R, F, capacity, variant, G, head_dim, schedule
    (2, 2, 2, 8, 4, 64, 32, 1024, "f32", 32, D,
     [("chunk", 45), ("steps", 3), ("chunk", 1), ("chunk", 100), ("steps", 40), ("chunk", 77),
      ("chunk", 31), ("steps", 2), ("chunk", 200), ("steps", 5)]),
    (1, 2, 2, 8, 4, 128, 128, 2048, "f16", 32, D,
     [("chunk", 300), ("steps", 20), ("chunk", 129), ("chunk", 500), ("steps", 130)]),
    (2, 1, 2, 4, 2, 0, 32, 512, "bf16", 32, D,
     [("chunk", 33), ("steps", 1), ("chunk", 64), ("chunk", 95), ("steps", 40), ("chunk", 7)]),
    (1, 2, 2, 8, 4, 128, 64, 1024, "f32", 64, D,
     [("chunk", 70), ("steps", 30), ("chunk", 250), ("steps", 3), ("chunk", 65)]),
    (1, 1, 2, 8, 4, 64, 32, 512, "f32", 32, 96,
     [("chunk", 50), ("steps", 20), ("chunk", 90), ("steps", 5)]),
]


@pytest.mark.parametrize("case", CHUNKED, ids=["f32", "meta16-F128", "bf16-R0", "G64", "D96"])
def test_chunked_prefill_matches_model(case):
    """Prompt chunks fed into a cache that already holds tokens (ragged
    chunk lengths, decode steps in between): the cache holds exactly what
    the model holds after the same tokens."""
    layers, batch, kvh, Hq, bits, R, F, cap, variant, G, Dh, sched = case
    _run_schedule(layers, batch, kvh, Hq, bits, R, F, cap, variant, sched, G, Dh, seed=7700 + R + G)


def test_prefill_of_8209_tokens_in_2048_token_chunks():
    """The Metal post's Generation 1 prompt of 8209 tokens, fed in 2048-token
    chunks (Lie #1: the runtime chunks prefill at 2048) with R = G = F = 32:
    8160 tokens flushed per layer, stores equal to the model's."""
    _run_schedule(2, 1, 8, 32, 4, 32, 32, 8192, "f32",
                  [("chunk", 2048)] * 4 + [("chunk", 17), ("steps", 2)], 32, D, seed=8209)


def test_full_store_is_reported_and_leaves_state_unchanged():
    """When the next flush would overflow the stores, end_step fails before
    launching anything and the cache keeps its state."""
    layers, batch, kvh, R, F, cap = 1, 1, 1, 32, 32, 64
    c = kivi.Cache(layers, batch, kvh, cap, 4, R, F)
    k0 = synth.kv_tensor(1, 127, keys=True, seed=1, device="cuda")
    v0 = synth.kv_tensor(1, 127, keys=False, seed=1, device="cuda")
    c.prefill(k0, v0)                      # Q = 64 = capacity, 63 fp16 tokens
    assert (c.n_quant, c.n_res) == (64, 63)
    kn = torch.zeros((1, D), dtype=torch.float16, device="cuda")
    c.append(0, kn, kn)
    state = (c.length, c.n_quant, c.n_res, c.head)
    with pytest.raises(kivi.KiviError):
        c.end_step()                       # 64 fp16 tokens would need a flush
    assert (c.length, c.n_quant, c.n_res, c.head) == state
    with pytest.raises(kivi.KiviError):
        c.append(0, kn, kn)                # the step is still open for layer 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("Dh,variant,S0", [(128, "f32", 70), (128, "f16", 70), (96, "bf16", 70), (64, "f32", 70),
                                           (128, "f32", 0)])
def test_fused_append_attend_matches_the_two_calls(Dh, variant, S0):
    """kivi_cache_append_attend against kivi_cache_append + kivi_cache_attend
    on two caches fed the same prompt (or none: the first step attends over
    its own token only) and tokens, through ring wraps and cross-layer
    flushes: every step's output bit-identical, and at the end the two device
    buffers (both zeroed before use) byte-identical, so the fused call wrote
    each token into its ring row exactly as the append."""
    layers, batch, kvh, Hq, bits, R, F, cap, steps = 3, 2, 2, 8, 4, 64, 32, 256, 75
    bf16 = variant == "bf16"
    meta = "f32" if bf16 else variant
    dtype = torch.bfloat16 if bf16 else torch.float16
    slabs, per = layers * batch * kvh, batch * kvh
    note(f"fused append+attend D={Dh} {variant} prompt={S0} layers={layers} R={R} F={F} steps={steps}")
    two = [kivi.Cache(layers, batch, kvh, cap, bits, R, F, meta=meta, dtype=dtype, head_dim=Dh) for _ in range(2)]
    for c in two:
        c.buffer.zero_()
    k0 = synth.kv_tensor(slabs, max(S0, 1), Dh, keys=True, seed=9900 + Dh, device="cuda", dtype=dtype)[:, :S0]
    v0 = synth.kv_tensor(slabs, max(S0, 1), Dh, keys=False, seed=9900 + Dh, device="cuda", dtype=dtype)[:, :S0]
    if S0:
        for c in two:
            c.prefill(k0, v0)
    ws = [kivi.attend_workspace(c.attend_workspace_bytes(Hq)) for c in two]
    for step in range(steps):
        kn = synth.kv_tensor(slabs, 1, Dh, keys=True, seed=9950 + step, device="cuda", dtype=dtype)[:, 0].contiguous()
        vn = synth.kv_tensor(slabs, 1, Dh, keys=False, seed=9950 + step, device="cuda", dtype=dtype)[:, 0].contiguous()
        q = synth.query(layers * batch, Hq, Dh, seed=9950 + step, device="cuda").to(dtype).view(layers, batch, Hq, Dh)
        for layer in range(layers):
            k1, v1 = kn[layer * per:(layer + 1) * per], vn[layer * per:(layer + 1) * per]
            two[0].append(layer, k1, v1)
            o_sep = two[0].attend(layer, q[layer].contiguous(), workspace=ws[0])
            o_fused = two[1].append_attend(layer, k1, v1, q[layer].contiguous(), workspace=ws[1])
            torch.cuda.synchronize()
            assert torch.equal(o_sep, o_fused), (step, layer)
        launches = [c.end_step() for c in two]
        assert launches[0] == launches[1]
        assert (two[0].length, two[0].n_quant) == (two[1].length, two[1].n_quant)
    torch.cuda.synchronize()
    assert two[0].length == S0 + steps and two[0].n_quant == (S0 + steps - R) // F * F
    assert torch.equal(two[0].buffer, two[1].buffer)
    # a second fused call on a layer that already appended this step is refused
    kn = torch.zeros((per, Dh), dtype=dtype, device="cuda")
    q = torch.zeros((batch, Hq, Dh), dtype=dtype, device="cuda")
    two[1].append_attend(0, kn, kn, q, workspace=ws[1])
    with pytest.raises(kivi.KiviError):
        two[1].append_attend(0, kn, kn, q, workspace=ws[1])
