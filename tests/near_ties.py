"""Quantization groups built to sit on the quantizer's rounding boundaries.

Each group of 32 values holds its minimum, its maximum and 30 elements x
whose binary32 quotient fl(fl(x - min) / scale), with scale = fl(fl(max -
min) / (2^bits - 1)), lies within 2^-12 of a half-integer (exact ties
included).  Those are the elements where a code computed any other way than
the quantizer's steps ([Metal post] "What we're actually optimizing"; "Three
ways to be off by one bit": ties to even) can come out one off, so a tensor
of such groups stresses every shortcut a kernel may take.

This module only selects inputs: the quotients above are numpy binary32
arithmetic used to decide which values to keep; the expected codes always
come from the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

NEAR = 2.0 ** -12


def _widen(bits16: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return bits16.view(np.float16).astype(np.float32)
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def _narrow(v: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest 16-bit value (ties to even) as bit patterns."""
    if fmt == "f16":
        return v.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _meta16(s: np.ndarray) -> np.ndarray:
    return s.astype(np.float16).astype(np.float32)


def near_tie_groups(n_groups: int, bits: int, seed: int, fmt: str = "f16", meta: str = "f32"):
    """-> (uint16 [n_groups][32] groups, number of near-tie elements)."""
    rng = np.random.default_rng(seed)
    L = np.float32((1 << bits) - 1)
    groups = []
    while len(groups) < n_groups:
        m = 2 * (n_groups - len(groups)) + 256
        # minima and ranges over four decades, up to the outlier channels' size
        mag = 10.0 ** rng.uniform(-3.0, 1.3, m)
        mn = _narrow(rng.standard_normal(m) * mag, fmt)
        mx = _narrow(_widen(mn, fmt).astype(np.float64) + (np.abs(rng.standard_normal(m)) * 2 + 0.05) * mag, fmt)
        mn32, mx32 = _widen(mn, fmt), _widen(mx, fmt)
        ok = np.isfinite(mx32) & (mx32 > mn32)
        mn, mx, mn32, mx32 = mn[ok], mx[ok], mn32[ok], mx32[ok]
        s = (mx32 - mn32) / L
        if meta == "f16":
            s = _meta16(s)
            keep = s >= np.float32(2.0 ** -14)
            mn, mx, mn32, mx32, s = mn[keep], mx[keep], mn32[keep], mx32[keep], s[keep]
        # candidates: the 16-bit values nearest to min + (k + 1/2) scale, and
        # their two neighbours (adjacent bit patterns)
        k = np.arange(int(L), dtype=np.float64) + 0.5
        target = mn32[:, None].astype(np.float64) + k[None, :] * s[:, None].astype(np.float64)
        c0 = _narrow(target, fmt).astype(np.int32)
        cands = np.concatenate([c0, c0 + 1, c0 - 1], axis=1).astype(np.uint16)
        cv = _widen(cands, fmt)
        with np.errstate(invalid="ignore", over="ignore"):
            u = (cv - mn32[:, None]) / s[:, None]
        dist = np.abs(u.astype(np.float64) - (np.floor(u.astype(np.float64)) + 0.5))
        good = np.isfinite(cv) & (cv > mn32[:, None]) & (cv < mx32[:, None]) & (dist <= NEAR)
        for i in np.nonzero(good.any(axis=1))[0]:
            xs = cands[i][good[i]]
            body = xs[rng.integers(0, len(xs), 30)]
            g = np.concatenate([[mn[i], mx[i]], body]).astype(np.uint16)
            groups.append(g[rng.permutation(32)])
            if len(groups) == n_groups:
                break
    return np.stack(groups), 30 * n_groups


def as_keys(groups: np.ndarray, BH: int, S: int, D: int = 128) -> np.ndarray:
    """[BH][S][D] whose key group (bh, g, d) -- tokens 32g..32g+31 of channel d
    -- is groups[(bh * S/32 + g) * D + d]."""
    return np.ascontiguousarray(groups.reshape(BH, S // 32, D, 32).transpose(0, 1, 3, 2).reshape(BH, S, D))


def as_values(groups: np.ndarray, BH: int, S: int, D: int = 128) -> np.ndarray:
    """[BH][S][D] whose value group (bh, s, j) -- channels 32j..32j+31 of token
    s -- is groups[(bh * S + s) * D/32 + j]."""
    return np.ascontiguousarray(groups.reshape(BH, S, D))
