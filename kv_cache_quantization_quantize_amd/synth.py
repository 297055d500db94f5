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

Every draw is counter-based, so a tensor is the same on any device and any
torch build (up to one ulp of the platform's double log/cos/sin, which the
rounding to 16 bits almost always hides; the exact tensor a test feeds the
HIP path is copied to the host for the oracle in any case):
  * element i of tensor ``tensor_id`` under ``seed`` (i the flat index in
    [BH][S][D] order) belongs to Box-Muller pair p = i // 2, whose two
    uniforms come from splitmix64(seed ^ tensor_id << 56 ^ 2p) and
    splitmix64(seed ^ tensor_id << 56 ^ (2p + 1)): the top 53 bits u as
    (u + 1) * 2^-53 in (0, 1] and u * 2^-53 in [0, 1);
  * with r = sqrt(-2 ln u1) and t = 2 pi u2 in double, element 2p is
    r cos t and element 2p + 1 is r sin t, rounded to float, multiplied by
    the outlier scale on outlier channels (in float), then rounded to fp16
    (or bfloat16) to nearest even;
  * the outlier channels of slab bh are the first ``n_outliers`` entries of
    a Fisher-Yates shuffle of 0 .. D-1 (j from D-1 down to 1 swaps j with
    r mod (j + 1)) whose r are the successive outputs of the splitmix64
    generator seeded with seed ^ 0xC0FFEE ^ bh.
splitmix64 is Steele, Lea and Flood's generator (state += 0x9E3779B97F4A7C15,
then the two xor-shift-multiply rounds and a final xor-shift); the counter
forms above apply it to a state of counter - 0x9E3779B97F4A7C15, so one
call mixes the counter itself.
"""
from __future__ import annotations

import math

import torch

VALUE_TENSOR = 1
KEY_TENSOR = 2
QUERY_TENSOR = 3
RESIDUAL_OFFSET = 16

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _signed(v: int) -> int:
    """A uint64 bit pattern as the int64 torch stores."""
    v &= _MASK64
    return v - (1 << 64) if v >= 1 << 63 else v


def _srl(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 tensors holding uint64 bits."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix(x: torch.Tensor) -> torch.Tensor:
    """splitmix64's output function of state x (int64 tensors, wrapping)."""
    x = (x ^ _srl(x, 30)) * _signed(_M1)
    x = (x ^ _srl(x, 27)) * _signed(_M2)
    return x ^ _srl(x, 31)


def splitmix64(counter: torch.Tensor) -> torch.Tensor:
    """One splitmix64 output per counter (int64 tensors holding uint64 bits):
    the generator's first output from state counter - golden."""
    return _mix(counter)


def splitmix64_int(v: int) -> int:
    """The same on a Python int (a reference the tests check the tensor form
    against)."""
    z = v & _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def outlier_channels(BH: int, D: int, seed: int, n_outliers: int = 4) -> torch.Tensor:
    """int64 [BH][n_outliers]: the scaled key channels of each slab."""
    out = torch.empty((BH, n_outliers), dtype=torch.int64)
    for bh in range(BH):
        state = (seed ^ 0xC0FFEE ^ bh) & _MASK64
        perm = list(range(D))
        for j in range(D - 1, 0, -1):
            state = (state + _GOLDEN) & _MASK64
            r = splitmix64_int(state) % (j + 1)
            perm[j], perm[r] = perm[r], perm[j]
        out[bh] = torch.tensor(perm[:n_outliers], dtype=torch.int64)
    return out


def normals(n: int, *, seed: int, tensor_id: int, first: int = 0, device="cpu") -> torch.Tensor:
    """float32 elements first .. first + n - 1 of the N(0, 1) stream of
    (seed, tensor_id)."""
    if n <= 0:
        return torch.empty(0, dtype=torch.float32, device=device)
    p0, p1 = first // 2, (first + n + 1) // 2               # Box-Muller pairs covering the range
    base = _signed((seed ^ (tensor_id << 56)) & _MASK64)
    pairs = torch.arange(p0, p1, dtype=torch.int64, device=device)
    b1 = splitmix64(base ^ (2 * pairs))
    b2 = splitmix64(base ^ (2 * pairs + 1))
    del pairs
    u1 = (_srl(b1, 11) + 1).to(torch.float64) * 2.0 ** -53
    u2 = _srl(b2, 11).to(torch.float64) * 2.0 ** -53
    del b1, b2
    r = torch.sqrt(-2.0 * torch.log(u1))
    t = (2.0 * math.pi) * u2
    del u1, u2
    z = torch.stack((r * torch.cos(t), r * torch.sin(t)), dim=1).reshape(-1)
    lo = first - 2 * p0
    return z[lo:lo + n].to(torch.float32)


def kv_tensor(BH: int, S: int, D: int = 128, *, keys: bool, seed: int,
              n_outliers: int = 4, outlier_scale: float = 10.0,
              device="cpu", tensor_id: int | None = None,
              slab_chunk: int = 8, dtype=torch.float16) -> torch.Tensor:
    """fp16 (or ``dtype``, e.g. bfloat16) [BH][S][D].  Drawn slab-chunk by
    slab-chunk to bound the temporaries (the long-context cache is 1.2e9
    elements per tensor)."""
    tid = tensor_id if tensor_id is not None else (KEY_TENSOR if keys else VALUE_TENSOR)
    out = torch.empty((BH, S, D), dtype=dtype, device=device)
    outl = outlier_channels(BH, D, seed, n_outliers) if (keys and n_outliers) else None
    per_slab = S * D
    for b0 in range(0, BH, slab_chunk):
        b1 = min(BH, b0 + slab_chunk)
        x = normals((b1 - b0) * per_slab, seed=seed, tensor_id=tid, first=b0 * per_slab,
                    device=device).view(b1 - b0, S, D)
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
    return normals(B * Hq * D, seed=seed, tensor_id=QUERY_TENSOR, device=device).view(B, Hq, D).half()


def residual(BH: int, R: int, D: int = 128, *, keys: bool, seed: int, device="cpu",
             n_outliers: int = 4, outlier_scale: float = 10.0) -> torch.Tensor:
    """fp16 residual window [BH][R][D]; keys share their slab's outliers."""
    return kv_tensor(BH, R, D, keys=keys, seed=seed, n_outliers=n_outliers,
                     outlier_scale=outlier_scale, device=device,
                     tensor_id=RESIDUAL_OFFSET + (KEY_TENSOR if keys else VALUE_TENSOR))
