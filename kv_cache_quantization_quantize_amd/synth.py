"""Seeded synthetic KV-cache inputs.

This module only draws inputs; it holds none of the quantizer's arithmetic,
so both the HIP path and the CPU oracle can be fed from it.

Recipe (the pages measure real model caches; these stand in for them with
the same shapes):
  * values: i.i.d. N(0, 1), rounded to fp16;
  * keys: i.i.d. N(0, 1) with ``n_outliers`` channels per (layer, kv-head)
    slab multiplied by ``outlier_scale`` before the fp16 rounding -- the
    pages motivate per-channel key quantization by a few key channels with
    consistently huge magnitudes (blog post "A 5.65x Metal Kernel That Made
    My LLM Exactly 0% Faster", section "What we're actually optimizing");
  * queries: i.i.d. N(0, 1) fp16.
The outlier channels of slab ``bh`` are the first ``n_outliers`` entries of
a seeded random permutation of the D channels drawn on the CPU, so they do
not depend on the device.  Normal draws use torch's generator of the target
device; the exact tensor a test feeds the HIP path is copied to the host for
the oracle, so the two never need to agree across devices.
"""
from __future__ import annotations

import torch

VALUE_TENSOR = 1
KEY_TENSOR = 2
QUERY_TENSOR = 3
RESIDUAL_OFFSET = 16


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def outlier_channels(BH: int, D: int, seed: int, n_outliers: int = 4) -> torch.Tensor:
    """int64 [BH][n_outliers]: the scaled key channels of each slab."""
    g = _gen("cpu", seed * 7919 + 0xC0FFEE)
    out = torch.empty((BH, n_outliers), dtype=torch.int64)
    for bh in range(BH):
        out[bh] = torch.randperm(D, generator=g)[:n_outliers]
    return out


def kv_tensor(BH: int, S: int, D: int = 128, *, keys: bool, seed: int,
              n_outliers: int = 4, outlier_scale: float = 10.0,
              device="cpu", tensor_id: int | None = None,
              slab_chunk: int = 8, dtype=torch.float16) -> torch.Tensor:
    """fp16 (or ``dtype``, e.g. bfloat16) [BH][S][D].  Drawn slab-chunk by
    slab-chunk to bound the float32 temporary (the long-context cache is
    1.2e9 elements per tensor)."""
    tid = tensor_id if tensor_id is not None else (KEY_TENSOR if keys else VALUE_TENSOR)
    out = torch.empty((BH, S, D), dtype=dtype, device=device)
    g = _gen(device, seed * 1_000_003 + tid)
    outl = outlier_channels(BH, D, seed, n_outliers) if (keys and n_outliers) else None
    for b0 in range(0, BH, slab_chunk):
        b1 = min(BH, b0 + slab_chunk)
        x = torch.randn((b1 - b0, S, D), generator=g, dtype=torch.float32, device=device)
        if outl is not None:
            mult = torch.ones((b1 - b0, 1, D), dtype=torch.float32)
            for i, bh in enumerate(range(b0, b1)):
                mult[i, 0, outl[bh]] = outlier_scale
            x.mul_(mult.to(device))
        out[b0:b1].copy_(x)
        del x
    return out


def query(B: int, Hq: int, D: int = 128, *, seed: int, device="cpu") -> torch.Tensor:
    """fp16 [B][Hq][D]."""
    g = _gen(device, seed * 1_000_003 + QUERY_TENSOR)
    return torch.randn((B, Hq, D), generator=g, dtype=torch.float32, device=device).half()


def residual(BH: int, R: int, D: int = 128, *, keys: bool, seed: int, device="cpu",
             n_outliers: int = 4, outlier_scale: float = 10.0) -> torch.Tensor:
    """fp16 residual window [BH][R][D]; keys share their slab's outliers."""
    return kv_tensor(BH, R, D, keys=keys, seed=seed, n_outliers=n_outliers,
                     outlier_scale=outlier_scale, device=device,
                     tensor_id=RESIDUAL_OFFSET + (KEY_TENSOR if keys else VALUE_TENSOR))
