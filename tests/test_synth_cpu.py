"""The seeded input generator (kv_cache_quantization_quantize_amd/synth.py):
splitmix64 against the generator's published output for seed 0, the tensor
form against the integer form, and the properties the recipe promises
(counter-based windows, N(0, 1) moments, outlier channels)."""
import random

import numpy as np
import torch

from kv_cache_quantization_quantize_amd import synth


def test_splitmix64_first_outputs_for_seed_zero():
    # the first three outputs of splitmix64 seeded with 0, as published with
    # the generator (Steele, Lea and Flood; Vigna's reference implementation)
    state, outs = 0, []
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) % 2 ** 64
        outs.append(synth.splitmix64_int(state))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_tensor_splitmix64_matches_the_integer_form():
    rng = random.Random(5)
    vals = [rng.getrandbits(64) for _ in range(4096)] + [0, 2 ** 63, 2 ** 64 - 1, 2 ** 63 - 1]
    got = synth.splitmix64(torch.tensor([synth._signed(v) for v in vals], dtype=torch.int64))
    assert [int(a) % 2 ** 64 for a in got.tolist()] == [synth.splitmix64_int(v) for v in vals]


def test_normals_are_counter_based_windows():
    whole = synth.normals(1001, seed=11, tensor_id=2)
    for first, n in ((0, 1), (1, 1), (1, 500), (333, 668), (1000, 1)):
        assert torch.equal(synth.normals(n, seed=11, tensor_id=2, first=first), whole[first:first + n])
    assert not torch.equal(synth.normals(1001, seed=12, tensor_id=2), whole)
    assert not torch.equal(synth.normals(1001, seed=11, tensor_id=3), whole)


def test_box_muller_pair_from_its_two_uniforms():
    """Elements 2p and 2p + 1 from the recipe written out in Python floats."""
    seed, tid, p = 1003, 1, 12345
    base = seed ^ (tid << 56)
    u1 = ((synth.splitmix64_int(base ^ (2 * p)) >> 11) + 1) * 2.0 ** -53
    u2 = (synth.splitmix64_int(base ^ (2 * p + 1)) >> 11) * 2.0 ** -53
    r = (-2.0 * np.log(u1)) ** 0.5
    want = np.array([r * np.cos(2 * np.pi * u2), r * np.sin(2 * np.pi * u2)], dtype=np.float32)
    got = synth.normals(2, seed=seed, tensor_id=tid, first=2 * p).numpy()
    assert np.allclose(got, want, rtol=0, atol=2e-7)


def test_normal_moments():
    x = synth.normals(2_000_000, seed=1003, tensor_id=1).double()
    assert abs(float(x.mean())) < 3e-3
    assert abs(float(x.std()) - 1.0) < 3e-3
    assert abs(float((x > 1.959964).double().mean()) - 0.025) < 1e-3


def test_outlier_channels_and_key_scaling():
    out = synth.outlier_channels(64, 128, seed=1003)
    assert out.shape == (64, 4)
    for row in out.tolist():
        assert len(set(row)) == 4 and all(0 <= c < 128 for c in row)
    assert len({tuple(r) for r in out.tolist()}) > 60              # slabs differ
    k = synth.kv_tensor(4, 256, keys=True, seed=1003).float()
    v = synth.kv_tensor(4, 256, keys=False, seed=1003).float()
    for bh in range(4):
        ch = out[bh].tolist()
        big = k[bh][:, ch].abs().mean()
        rest = np.delete(k[bh].numpy(), ch, axis=1)
        assert 6.0 < float(big) < 10.0 and 0.6 < float(np.abs(rest).mean()) < 1.0
    assert 0.6 < float(v.abs().mean()) < 1.0
    # the same draws at another chunking of the slabs
    assert torch.equal(synth.kv_tensor(5, 64, keys=True, seed=9, slab_chunk=2),
                       synth.kv_tensor(5, 64, keys=True, seed=9, slab_chunk=8))
