"""The calibration kernels (include/kivi_calib.h) move exactly the bytes
their traffic shape names, since their rates serve as bandwidth ceilings:
the copy reproduces its source, the write fills every 16-byte vector with
its pattern, the mix writes the first 3/8 of the source's size in its three
regions (each vector the XOR of one lane's eight loads) and nothing past
it, and the read leaves its sink alone unless a thread's fold equals the
sentinel.  Sizes include a ragged last workgroup (not a multiple of 16 KiB)
and ragged last mix tiles.  Exact comparisons."""
import numpy as np
import pytest
import torch

from gpu_util import note
from kv_cache_quantization_quantize_amd import kivi

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BLOCK, VECS = 256, 4                 # threads per workgroup, 16-byte vectors per thread
CHUNK = BLOCK * VECS                 # vectors per workgroup
SIZES = [16 * 37, 16384 * 5 + 16 * 37, (1 << 20) + 48, 16384 * 64]


def _src(n_bytes: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, (n_bytes,), dtype=torch.uint8, generator=g)


def _thread_folds(src: np.ndarray) -> np.ndarray:
    """[blocks, BLOCK, 4] uint32: the XOR of each thread's VECS loads (zero
    past the end), thread t of block b loading vectors b*CHUNK + t + BLOCK*u."""
    v = src.view(np.uint32).reshape(-1, 4)
    n_vec = v.shape[0]
    blocks = (n_vec + CHUNK - 1) // CHUNK
    pad = np.zeros((blocks * CHUNK, 4), np.uint32)
    pad[:n_vec] = v
    per = pad.reshape(blocks, VECS, BLOCK, 4)
    return np.bitwise_xor.reduce(per, axis=1)


@pytest.mark.parametrize("n", SIZES)
def test_copy_reproduces_its_source(n):
    note(f"calib copy n={n}")
    src = _src(n, 1).cuda()
    dst = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    kivi.calib_copy(src, dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert bool((dst[n:] == 0xA5).all())


@pytest.mark.parametrize("n", SIZES)
def test_write_fills_every_vector(n):
    note(f"calib write n={n}")
    dst = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    kivi.calib_write(dst[:n])
    torch.cuda.synchronize()
    got = dst[:n].cpu().numpy().view(np.uint32).reshape(-1, 4)
    i = np.arange(got.shape[0], dtype=np.uint32)
    pat = np.uint32(0x5A5A5A5A)
    want = np.stack([np.full_like(i, pat), pat ^ i, np.full_like(i, pat), np.zeros_like(i)], axis=1)
    assert np.array_equal(got, want)
    assert bool((dst[n:] == 0xA5).all())


def _mix_expected(src: np.ndarray) -> np.ndarray:
    """dst of the flush-shaped mix: wave t folds lanes l's loads of source
    vectors 512t + l + 64u (u < 8) and writes the fold of lane k mod 64 to
    codes[128t + k], of lane k mod 32 to scale[32t + k] and of lane 32 +
    (k mod 32) to zero[32t + k], the regions holding n/4, n/16 and the rest
    of 3n/8 vectors (the last tile's counts absorb a ragged end)."""
    v = src.view(np.uint32).reshape(-1, 4)
    n = v.shape[0]
    tiles = (n + 511) // 512
    pad = np.zeros((tiles * 512, 4), np.uint32)
    pad[:n] = v
    lanes = np.bitwise_xor.reduce(pad.reshape(tiles, 8, 64, 4), axis=1)     # [tile, lane, 4]
    m, mc, ms = n * 3 // 8, n // 4, n // 16
    mz = m - mc - ms
    out = np.zeros((m, 4), np.uint32)
    for start, size, stride, lane_of in ((0, mc, 128, lambda k: k % 64),              # codes
                                         (mc, ms, 32, lambda k: k % 32),              # scale
                                         (mc + ms, mz, 32, lambda k: 32 + k % 32)):   # zero
        j = np.arange(size)
        t = np.minimum(j // stride, tiles - 1)          # the last tile takes any overflow
        k = j - t * stride
        out[start + j] = lanes[t, lane_of(k)]
    return out


@pytest.mark.parametrize("n", SIZES + [16 * 511, 16 * (512 * 3 + 511)])
def test_mix_writes_three_eighths(n):
    note(f"calib mix n={n}")
    src_h = _src(n, 2)
    src = src_h.cuda()
    n_out = (n // 16) * 3 // 8 * 16
    dst = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    kivi.calib_mix(src, dst)
    torch.cuda.synchronize()
    got = dst[:n_out].cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(got, _mix_expected(src_h.numpy()))
    assert bool((dst[n_out:] == 0xA5).all())


@pytest.mark.parametrize("n", SIZES)
def test_read_writes_only_on_a_sentinel_match(n):
    note(f"calib read n={n}")
    src_h = _src(n, 3)
    sink = torch.full((16,), 0xA5, dtype=torch.uint8, device="cuda")
    kivi.calib_read(src_h.cuda(), sink)
    torch.cuda.synchronize()
    f = _thread_folds(src_h.numpy())
    folds = f[..., 0] ^ f[..., 1] ^ f[..., 2] ^ f[..., 3]
    got = sink.cpu().numpy()
    if (folds == np.uint32(0x9E3779B9)).any():
        assert got[:4].view(np.uint32)[0] == 0x9E3779B9
        assert bool((got[4:] == 0xA5).all())
    else:
        assert bool((got == 0xA5).all())
