"""Exact-rational emulation of binary16/binary32 rounding (test helper).

Every value is a ``fractions.Fraction``; each IEEE operation is the exact
result followed by an explicit round-to-nearest-even onto the format's grid,
written from the formats' definitions.  It shares no arithmetic with the C
oracle (which uses the host's float unit) and is slow: tiny inputs only.
"""
from __future__ import annotations

from fractions import Fraction
import math
import struct


def _floor_log2(r: Fraction) -> int:
    """e with 2**e <= r < 2**(e+1), for r > 0."""
    e = r.numerator.bit_length() - r.denominator.bit_length()
    if Fraction(2) ** e > r:
        e -= 1
    if Fraction(2) ** (e + 1) <= r:
        e += 1
    return e


def _rhe(n: Fraction) -> int:
    """Round a non-negative rational to an integer, ties to even."""
    fl = n.numerator // n.denominator
    fr = n - fl
    if fr > Fraction(1, 2):
        return fl + 1
    if fr < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _round(r: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Nearest-even rounding of r onto a binary format with ``mant_bits``
    fraction bits and minimum normal exponent ``emin`` (no overflow)."""
    if r == 0:
        return Fraction(0)
    s = -1 if r < 0 else 1
    a = abs(r)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - mant_bits)
    return s * _rhe(a / quantum) * quantum


def rnd32(r: Fraction) -> Fraction:
    return _round(Fraction(r), 23, -126)


def rnd16(r: Fraction) -> Fraction:
    return _round(Fraction(r), 10, -14)


def f16_value(bits: int) -> Fraction:
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    assert e != 31, "finite inputs only"
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f) * Fraction(2) ** (e - 25)


def f16_bits(v: Fraction) -> int:
    """Encode a value already on the binary16 grid (|v| <= 65504)."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    if a < Fraction(1, 1 << 14):
        n = a * (1 << 24)
        assert n.denominator == 1
        return sign | int(n)
    e = _floor_log2(a)
    n = a / Fraction(2) ** (e - 10)
    assert n.denominator == 1 and 1024 <= n < 2048
    return sign | ((e + 15) << 10) | (int(n) - 1024)


def rnd16_bits(r: Fraction) -> int:
    """binary16 encoding of RN16(r), keeping the sign of a result that
    rounds to zero (IEEE: the rounded result carries the operand's sign)."""
    r = Fraction(r)
    bits = f16_bits(abs(rnd16(r)))
    return bits | 0x8000 if r < 0 else bits


def rndbf16(r: Fraction) -> Fraction:
    return _round(Fraction(r), 7, -126)


def bf16_value(bits: int) -> Fraction:
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 255, "finite inputs only"
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** -133
    return sign * Fraction(128 + f) * Fraction(2) ** (e - 134)


def bf16_bits(v: Fraction) -> int:
    """Encode a value already on the bfloat16 grid."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    if a < Fraction(2) ** -126:
        n = a * Fraction(2) ** 133
        assert n.denominator == 1
        return sign | int(n)
    e = _floor_log2(a)
    n = a / Fraction(2) ** (e - 7)
    assert n.denominator == 1 and 128 <= n < 256
    return sign | ((e + 127) << 7) | (int(n) - 128)


def rndbf16_bits(r: Fraction) -> int:
    r = Fraction(r)
    bits = bf16_bits(abs(rndbf16(r)))
    return bits | 0x8000 if r < 0 else bits


def f32_bits(v: Fraction) -> int:
    """Bit pattern of a value already on the binary32 grid."""
    f = float(v)  # exact: v is representable in binary32, hence in binary64
    return struct.unpack("<I", struct.pack("<f", f))[0]


def quantize_group(xbits, bits: int, *, ties="even", quotient="fp32",
                   recon_fma=False, fmt="f16", meta="f32"):
    """Emulate one group.  The keyword arguments select deliberately wrong
    variants (used to show that a fixture discriminates):
      ties="away"          round half away from zero instead of half to even
      quotient="exact"     round the exact rational (x-zero)/scale, not its
                           binary32 rounding
      quotient="rcp"       binary32 (x-zero) * binary32(1/scale)
      recon_fma=True       one rounding for q*scale+zero (a fused multiply-add)
      fmt="bf16"           inputs and reconstructions in bfloat16
      meta="f16"           scale and zero stored as binary16 (the reading:
                           codes and reconstruction use the stored values)
      meta="f16_store_only"  wrong: codes from the binary32 scale, only the
                           reconstruction from the binary16 one
    Returns (scale, zero, codes, recon_bits) with scale/zero as Fractions."""
    value, to_bits = (f16_value, rnd16_bits) if fmt == "f16" else (bf16_value, rndbf16_bits)
    xs = [value(b) for b in xbits]
    mn, mx = min(xs), max(xs)
    levels = (1 << bits) - 1
    rng = rnd32(mx - mn)
    scale = rnd32(rng / levels)
    zero = mn
    code_scale = scale
    if meta in ("f16", "f16_store_only"):
        scale, zero = rnd16(scale), rnd16(zero)
        code_scale = scale if meta == "f16" else code_scale
    codes, recon = [], []
    for x in xs:
        if code_scale == 0:
            q = 0
        else:
            t = rnd32(x - zero)
            if quotient == "fp32":
                u = rnd32(t / code_scale)
            elif quotient == "exact":
                u = t / code_scale
            elif quotient == "rcp":
                u = rnd32(t * rnd32(1 / code_scale))
            else:
                raise ValueError(quotient)
            if ties == "even":
                q = _rhe(u) if u >= 0 else -_rhe(-u)
            else:
                q = math.floor(u + Fraction(1, 2)) if u >= 0 else -math.floor(-u + Fraction(1, 2))
            q = min(max(q, 0), levels)
        if recon_fma:
            r = rnd32(q * scale + zero)
        else:
            r = rnd32(rnd32(q * scale) + zero)
        codes.append(q)
        recon.append(to_bits(r))
    return scale, zero, codes, recon
