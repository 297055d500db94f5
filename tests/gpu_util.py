"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same input bytes, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from kv_cache_quantization_quantize_amd import kivi

CODE_SENTINEL = 0x5A5A5A5A
META_SENTINEL = -7.25
F16_SENTINEL = 0x7BFF   # 65504: never a reconstruction of these inputs


def note(msg: str) -> None:
    """Name the case before a GPU step, so a crash still says what ran."""
    print(msg, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def device_store(kind: int, BH: int, cap: int, bits: int) -> kivi.Store:
    st = kivi.Store(kind, BH, cap, bits)
    st.codes.fill_(CODE_SENTINEL)
    st.scale.fill_(META_SENTINEL)
    st.zero.fill_(META_SENTINEL)
    return st


def host_store(kind: int, BH: int, cap: int, bits: int) -> oracle.Store:
    okind = oracle.KEYS if kind == kivi.KIVI_KEYS else oracle.VALUES
    return oracle.Store(okind, BH, cap, 128, bits, 32, fill_codes=CODE_SENTINEL, fill_meta=META_SENTINEL)


def store_to_host(st: kivi.Store, slabs=None):
    sel = slice(None) if slabs is None else slabs
    return (st.codes[sel].cpu().numpy().view(np.uint32), st.scale[sel].cpu().numpy(),
            st.zero[sel].cpu().numpy())


def assert_store_equal(gpu: kivi.Store, host: oracle.Store, slabs=None, what=""):
    codes, scale, zero = store_to_host(gpu, slabs)
    hsel = slice(None) if slabs is None else slabs
    hc, hs, hz = host.codes[hsel], host.scale[hsel], host.zero[hsel]
    if not np.array_equal(codes, hc):
        bad = np.argwhere(codes != hc)
        raise AssertionError(f"{what}: {len(bad)} code words differ, first at {bad[0].tolist()}: "
                             f"gpu {codes[tuple(bad[0])]:#010x} oracle {hc[tuple(bad[0])]:#010x}")
    # compare metadata as bit patterns (the sentinel and +0 must match
    # exactly); a binary16 host store holds binary16 values, so its
    # conversion to binary16 bits is exact
    if getattr(gpu, "meta", "f32") == "f16":
        assert host.meta == "f16"
        gs, gz = scale.view(np.uint16), zero.view(np.uint16)
        hs, hz = oracle.f32_to_f16(hs), oracle.f32_to_f16(hz)
    else:
        gs, gz, hs, hz = scale.view(np.uint32), zero.view(np.uint32), hs.view(np.uint32), hz.view(np.uint32)
    if not np.array_equal(gs, hs):
        bad = np.argwhere(gs != hs)
        raise AssertionError(f"{what}: {len(bad)} scales differ, first at {bad[0].tolist()}: "
                             f"gpu {gs[tuple(bad[0])]:#x} oracle {hs[tuple(bad[0])]:#x}")
    if not np.array_equal(gz, hz):
        bad = np.argwhere(gz != hz)
        raise AssertionError(f"{what}: {len(bad)} zeros differ, first at {bad[0].tolist()}")


def assert_u16_equal(got: np.ndarray, want: np.ndarray, what=""):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} fp16 values differ, first at {bad[0].tolist()}: "
                             f"gpu {got[tuple(bad[0])]:#06x} oracle {want[tuple(bad[0])]:#06x}")
