"""CPU oracle for the KIVI flush, dequantize and dequantize-then-attend.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``kv_cache_quantization_quantize_amd``) never imports it, and it never imports
the product: the two share no code.

The arithmetic lives in ``kivi_oracle.c`` (plain single-threaded C, built with
``-ffp-contract=off``); this module only marshals numpy arrays into it.

Parity status of each function (what pins it is in ``tests/test_oracle_*.py``):
  f16_to_f32 / f32_to_f16 ..... pinned (exhaustive against numpy's IEEE codec)
  bf16_to_f32 / f32_to_bf16 ... pinned (all 65536 patterns and whole fp32
                                exponents against torch's bfloat16 codec)
  quantize_group .............. pinned (hand-worked groups, invariants, brute
                                force against an exact-rational emulation)
  quantize_keys / _values ..... pinned (layout fixtures, per-group reduction to
                                quantize_group, axis-discriminating fixtures);
                                bf16 inputs: hand-worked groups and brute force
                                against the exact-rational emulation
  dequantize .................. pinned (hand-worked reconstructions, identity
                                with the flush's own reconstruction)
  decode_attend ............... pinned (closed forms: one token, equal scores,
                                shift invariance; torch float64 SDPA when the
                                store is empty)
  decode_attend_varlen ........ pinned (equal lengths reproduce decode_attend;
                                each sequence equals its own batch of one and
                                does not depend on the others; empty -> 0)
  flush_count ................. pinned (the flush/layer figures of the
                                Generation 1 table)
  CacheModel .................. pinned (incremental stores equal one flush of
                                the same prefix; token split per step checked
                                with torch float64 SDPA; counts follow the rule)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "kivi_oracle.c")

KEYS = 0
VALUES = 1
FMT = {"f16": 0, "bf16": 1}        # 16-bit storage format of inputs and reconstructions
META = {"f32": 0, "f16": 1}       # storage format of a store's scale and zero

# -ffp-contract=off keeps a*b+c as two roundings; no -ffast-math anywhere.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc; always recompiles."""
    cmd = ["gcc", *CFLAGS, "-o", LIB_PATH + ".tmp", SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def lib():
    """Load the built oracle; build it only when nothing is built yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            # building starts gcc as a child process, which a process that has
            # already set up a GPU must not do: build beforehand instead
            torch = sys.modules.get("torch")
            if torch is not None and torch.cuda.is_initialized():
                raise RuntimeError(f"{LIB_PATH} is not built; run oracle.build() before any GPU work")
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
        L.orc_f32_to_f16_array.argtypes = [_f32p, _u16p, _i64]
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_bf16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
        L.orc_f32_to_bf16_array.argtypes = [_f32p, _u16p, _i64]
        L.orc_quantize_group_fmt.argtypes = [_u16p, _int, _int, _int, _f32p, _f32p, _u8p, _u16p]
        L.orc_dequantize_one_fmt.argtypes = [ctypes.c_uint32, ctypes.c_float, ctypes.c_float, _int]
        L.orc_dequantize_one_fmt.restype = ctypes.c_uint16
        L.orc_quantize_group.argtypes = [_u16p, _int, _int, _f32p, _f32p, _u8p, _u16p]
        L.orc_dequantize_one.argtypes = [ctypes.c_uint32, ctypes.c_float, ctypes.c_float]
        L.orc_dequantize_one.restype = ctypes.c_uint16
        flush_args = [_u16p, _i64, _i64, _i64, _i64, _int, _int,
                      _u32p, _i64, _f32p, _f32p, _i64, _i64, _u16p, _i64]
        L.orc_quantize_keys.argtypes = flush_args
        L.orc_quantize_values.argtypes = flush_args
        L.orc_quantize_keys.restype = _int
        L.orc_quantize_values.restype = _int
        L.orc_quantize_group_meta.argtypes = [_u16p, _int, _int, _int, _int, _f32p, _f32p, _u8p,
                                              _u16p]
        L.orc_quantize_keys_meta.argtypes = flush_args + [_int, _int]
        L.orc_quantize_values_meta.argtypes = flush_args + [_int, _int]
        L.orc_quantize_keys_meta.restype = _int
        L.orc_quantize_values_meta.restype = _int
        L.orc_quantize_keys_fmt.argtypes = flush_args + [_int]
        L.orc_quantize_values_fmt.argtypes = flush_args + [_int]
        L.orc_quantize_keys_fmt.restype = _int
        L.orc_quantize_values_fmt.restype = _int
        L.orc_dequantize.argtypes = [_int, _u32p, _i64, _f32p, _f32p, _i64,
                                     _i64, _i64, _int, _int, _i64, _i64, _u16p, _i64]
        L.orc_dequantize.restype = _int
        L.orc_dequantize_fmt.argtypes = L.orc_dequantize.argtypes + [_int]
        L.orc_dequantize_fmt.restype = _int
        L.orc_decode_attend.argtypes = [
            _u16p, _i64, _int, _int, _i64,
            _u32p, _f32p, _f32p, _u32p, _f32p, _f32p,
            _i64, _i64, _i64, _int, _int, _i64,
            _u16p, _u16p, _i64, _i64, ctypes.c_double, _f64p]
        L.orc_decode_attend.restype = _int
        L.orc_decode_attend_fmt.argtypes = L.orc_decode_attend.argtypes + [_int]
        L.orc_decode_attend_fmt.restype = _int
        L.orc_flush_count.argtypes = [_i64, _i64, _i64]
        L.orc_flush_count.restype = _i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_u16(x) -> np.ndarray:
    """fp16 bit patterns as a contiguous uint16 array (accepts float16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return x


# ------------------------------------------------------------------ codec
def f16_to_f32(h) -> np.ndarray:
    h = _as_u16(h)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


def f32_to_f16(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_f16_array(_ptr(f, ctypes.c_float), _ptr(out, ctypes.c_uint16), f.size)
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = _as_u16(h)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


def f32_to_bf16(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(f, ctypes.c_float), _ptr(out, ctypes.c_uint16), f.size)
    return out


# ------------------------------------------------------------------ groups
def quantize_group(x, bits: int, fmt: str = "f16", meta: str = "f32"):
    """-> (scale fp32, zero fp32, codes uint8[n], recon bits uint16[n]) for
    n values stored as fp16 or bf16 bit patterns (``fmt``).  With ``meta``
    "f16" the scale and zero are the binary16-rounded values (widened) that
    the codes and the reconstruction were taken with."""
    x = _as_u16(x).reshape(-1)
    n = x.size
    assert meta == "f32" or fmt == "f16", "binary16 metadata is for fp16 inputs"
    sc = np.zeros(1, np.float32)
    ze = np.zeros(1, np.float32)
    q = np.zeros(n, np.uint8)
    rec = np.zeros(n, np.uint16)
    lib().orc_quantize_group_meta(_ptr(x, ctypes.c_uint16), n, bits, FMT[fmt], META[meta],
                                  _ptr(sc, ctypes.c_float), _ptr(ze, ctypes.c_float),
                                  _ptr(q, ctypes.c_uint8), _ptr(rec, ctypes.c_uint16))
    return sc[0], ze[0], q, rec


def dequantize_one(q: int, scale, zero, fmt: str = "f16") -> int:
    return int(lib().orc_dequantize_one_fmt(int(q), float(np.float32(scale)), float(np.float32(zero)),
                                            FMT[fmt]))


# ------------------------------------------------------------------ store
class Store:
    """Host packed store in the documented layout (see kivi_oracle.h).

    ``meta`` is the storage format of scale and zero ("f32" or "f16"); the
    arrays are float32 either way, holding the binary16 values widened for
    "f16" (``meta_bits`` gives their bit patterns)."""

    def __init__(self, kind: int, BH: int, cap: int, D: int = 128, bits: int = 4,
                 G: int = 32, fill_codes: int = 0, fill_meta: float = 0.0, meta: str = "f32"):
        assert kind in (KEYS, VALUES) and meta in META
        self.kind, self.BH, self.cap, self.D, self.bits, self.G = kind, BH, cap, D, bits, G
        self.meta = meta
        self.words = D * bits // 32
        self.codes = np.full((BH, cap, self.words), fill_codes, np.uint32)
        if kind == KEYS:
            meta_shape = (BH, (cap + G - 1) // G, D)     # a ragged last group has its pair too
        else:
            meta_shape = (BH, cap, (D + G - 1) // G)
        self.scale = np.full(meta_shape, fill_meta, np.float32)
        self.zero = np.full(meta_shape, fill_meta, np.float32)

    def slabs(self, lo: int, hi: int) -> "Store":
        """Slabs [lo, hi) as a store of their own (views, not copies)."""
        sub = Store.__new__(Store)
        sub.kind, sub.BH, sub.cap, sub.D, sub.bits, sub.G = self.kind, hi - lo, self.cap, self.D, \
            self.bits, self.G
        sub.meta = self.meta
        sub.words = self.words
        sub.codes, sub.scale, sub.zero = self.codes[lo:hi], self.scale[lo:hi], self.zero[lo:hi]
        return sub

    @property
    def codes_bh_stride(self) -> int:
        return self.codes.shape[1] * self.codes.shape[2]

    @property
    def meta_bh_stride(self) -> int:
        return self.scale.shape[1] * self.scale.shape[2]

    def meta_bits(self):
        """(scale, zero) as binary16 bit patterns (exact for an "f16" store)."""
        assert self.meta == "f16"
        return f32_to_f16(self.scale), f32_to_f16(self.zero)


def _flush(fn, x, store: Store, dst_token: int, want_recon: bool, fmt: str):
    x = _as_u16(x)
    BH, S, D = x.shape
    assert BH == store.BH and D == store.D
    recon = np.zeros((BH, S, D), np.uint16) if want_recon else None
    rc = fn(_ptr(x, ctypes.c_uint16), BH, S, D, S * D, store.bits, store.G,
            _ptr(store.codes, ctypes.c_uint32), store.codes_bh_stride,
            _ptr(store.scale, ctypes.c_float), _ptr(store.zero, ctypes.c_float),
            store.meta_bh_stride, dst_token,
            _ptr(recon, ctypes.c_uint16), S * D, FMT[fmt], META[store.meta])
    if rc != 0:
        raise ValueError("oracle rejected the flush arguments")
    return recon


def quantize_keys(x, store: Store, dst_token: int = 0, want_recon: bool = True, fmt: str = "f16"):
    """Per-channel key flush of x[BH][S][D] (fp16 or bf16 bits, ``fmt``) into
    ``store`` at ``dst_token``; the reconstruction comes back in ``fmt``."""
    assert store.kind == KEYS
    return _flush(lib().orc_quantize_keys_meta, x, store, dst_token, want_recon, fmt)


def quantize_values(x, store: Store, dst_token: int = 0, want_recon: bool = True, fmt: str = "f16"):
    """Per-token value flush of x[BH][S][D] (fp16 or bf16 bits, ``fmt``) into
    ``store`` at ``dst_token``; the reconstruction comes back in ``fmt``."""
    assert store.kind == VALUES
    return _flush(lib().orc_quantize_values_meta, x, store, dst_token, want_recon, fmt)


def dequantize(store: Store, t0: int, n: int, fmt: str = "f16") -> np.ndarray:
    """Reconstruction of tokens [t0, t0 + n) as fp16 or bf16 bits (``fmt``)."""
    out = np.zeros((store.BH, n, store.D), np.uint16)
    rc = lib().orc_dequantize_fmt(store.kind, _ptr(store.codes, ctypes.c_uint32),
                                  store.codes_bh_stride, _ptr(store.scale, ctypes.c_float),
                                  _ptr(store.zero, ctypes.c_float), store.meta_bh_stride,
                                  store.BH, store.D, store.bits, store.G, t0, n,
                                  _ptr(out, ctypes.c_uint16), n * store.D, FMT[fmt])
    if rc != 0:
        raise ValueError("oracle rejected the dequantize arguments")
    return out


def decode_attend(q, B: int, Hq: int, Hkv: int, kstore: Store | None, vstore: Store | None,
                  n_quant: int, k_res, v_res, n_res: int,
                  softmax_scale: float | None = None, fmt: str = "f16") -> np.ndarray:
    """float64 [B][Hq][D] = softmax(q K^T * scale) V over store + residual.

    ``k_res``/``v_res`` are [B*Hkv][R][D] with n_res <= R used rows; q, the
    residual and the store's reconstruction are fp16 or bf16 (``fmt``)."""
    q = _as_u16(q).reshape(B, Hq, -1)
    D = q.shape[2]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D), np.float64)
    if n_quant > 0:
        ks, vs = kstore, vstore
        assert ks.codes_bh_stride == vs.codes_bh_stride and ks.bits == vs.bits
        args = (_ptr(ks.codes, ctypes.c_uint32), _ptr(ks.scale, ctypes.c_float),
                _ptr(ks.zero, ctypes.c_float), _ptr(vs.codes, ctypes.c_uint32),
                _ptr(vs.scale, ctypes.c_float), _ptr(vs.zero, ctypes.c_float),
                ks.codes_bh_stride, ks.meta_bh_stride, vs.meta_bh_stride, ks.bits, ks.G)
    else:
        z32, zf = np.zeros(1, np.uint32), np.zeros(1, np.float32)
        args = (_ptr(z32, ctypes.c_uint32), _ptr(zf, ctypes.c_float), _ptr(zf, ctypes.c_float),
                _ptr(z32, ctypes.c_uint32), _ptr(zf, ctypes.c_float), _ptr(zf, ctypes.c_float),
                0, 0, 0, 4, 32)
    if n_res > 0:
        k_res = _as_u16(k_res)
        v_res = _as_u16(v_res)
        res_stride = k_res.shape[1] * k_res.shape[2]
        assert v_res.shape == k_res.shape
    else:
        k_res = v_res = np.zeros(1, np.uint16)
        res_stride = 0
    rc = lib().orc_decode_attend_fmt(_ptr(q, ctypes.c_uint16), B, Hq, Hkv, D, *args, n_quant,
                                     _ptr(k_res, ctypes.c_uint16), _ptr(v_res, ctypes.c_uint16),
                                     res_stride, n_res, float(softmax_scale),
                                     _ptr(out, ctypes.c_double), FMT[fmt])
    if rc != 0:
        raise ValueError("oracle rejected the attend arguments")
    return out


def decode_attend_varlen(q, B: int, Hq: int, Hkv: int, kstore: Store | None,
                         vstore: Store | None, n_quant, max_n_quant: int, k_res, v_res,
                         n_res, max_n_res: int, softmax_scale: float | None = None,
                         fmt: str = "f16") -> np.ndarray:
    """float64 [B][Hq][D]: sequence b is ``decode_attend`` of a batch of one over
    its own slabs b*Hkv .. b*Hkv + Hkv - 1, with n_quant[b] store tokens and
    n_res[b] residual tokens, each clamped to [0, max]; a sequence left with no
    token gets zeros (attention over an empty set is undefined)."""
    q = _as_u16(q).reshape(B, Hq, -1)
    out = np.zeros((B, Hq, q.shape[2]), np.float64)
    if max_n_res > 0:
        k_res, v_res = _as_u16(k_res), _as_u16(v_res)
    for b in range(B):
        nq = min(max(int(n_quant[b]), 0), max_n_quant)
        nr = min(max(int(n_res[b]), 0), max_n_res)
        if nq + nr == 0:
            continue
        lo, hi = b * Hkv, (b + 1) * Hkv
        out[b] = decode_attend(q[b:b + 1], 1, Hq, Hkv,
                               kstore.slabs(lo, hi) if nq else None,
                               vstore.slabs(lo, hi) if nq else None, nq,
                               k_res[lo:hi] if nr else None, v_res[lo:hi] if nr else None, nr,
                               softmax_scale, fmt)[0]
    return out


def flush_count(S: int, R: int, G: int) -> int:
    return int(lib().orc_flush_count(S, R, G))


class CacheModel:
    """The decode loop's cache as a plain model: every slab keeps all of its
    fp16 tokens in order; after the prompt and after every step the oldest
    flush_count(S, R, F) tokens of a sequence of S tokens are in the stores
    (whole units of F older than the newest R, the rule of ``flush_count``
    with F in place of G), flushed by ``quantize_keys`` / ``quantize_values``
    as they cross that line.  A step's attention (``decode_attend``) sees the
    store tokens and every later token, the step's own one included, in
    order.  Slab s = (layer * batch + b) * kv_heads + h."""

    def __init__(self, layers: int, batch: int, kv_heads: int, capacity: int, bits: int = 4,
                 R: int = 128, F: int = 32, D: int = 128, meta: str = "f32", fmt: str = "f16",
                 G: int = 32):
        self.layers, self.batch, self.kv_heads, self.R, self.F, self.D = layers, batch, kv_heads, R, F, D
        self.fmt = fmt
        self.slabs = layers * batch * kv_heads
        self.kstore = Store(KEYS, self.slabs, capacity, D, bits, G, meta=meta)
        self.vstore = Store(VALUES, self.slabs, capacity, D, bits, G, meta=meta)
        self.k = np.zeros((self.slabs, 0, D), np.uint16)
        self.v = np.zeros((self.slabs, 0, D), np.uint16)
        self.n_quant = 0

    @property
    def length(self) -> int:
        return self.k.shape[1]

    def _flush_to_rule(self):
        Q = flush_count(self.length, self.R, self.F)
        if Q > self.n_quant:
            quantize_keys(np.ascontiguousarray(self.k[:, self.n_quant:Q]), self.kstore, self.n_quant,
                          want_recon=False, fmt=self.fmt)
            quantize_values(np.ascontiguousarray(self.v[:, self.n_quant:Q]), self.vstore, self.n_quant,
                            want_recon=False, fmt=self.fmt)
            self.n_quant = Q

    def prefill(self, k, v):
        """k, v 16-bit [slabs][S][D]: S more prompt tokens of every layer and
        sequence (the whole prompt, or the next chunk of it), appended to the
        tokens the model holds; then the rule flushes what it calls for."""
        self.k = np.concatenate([self.k, _as_u16(k)], axis=1)
        self.v = np.concatenate([self.v, _as_u16(v)], axis=1)
        self._flush_to_rule()

    def step(self, k_new, v_new, q, Hq: int) -> np.ndarray:
        """k_new, v_new [slabs][D] (this step's token of every slab) and q
        [layers][batch][Hq][D], 16-bit in the model's format.  Returns float64
        [layers][batch][Hq][D]."""
        self.k = np.concatenate([self.k, _as_u16(k_new)[:, None, :]], axis=1)
        self.v = np.concatenate([self.v, _as_u16(v_new)[:, None, :]], axis=1)
        q = _as_u16(q)
        per = self.batch * self.kv_heads
        out = np.zeros((self.layers, self.batch, Hq, self.D), np.float64)
        nq, nr = self.n_quant, self.length - self.n_quant
        for layer in range(self.layers):
            lo, hi = layer * per, (layer + 1) * per
            out[layer] = decode_attend(q[layer], self.batch, Hq, self.kv_heads,
                                       self.kstore.slabs(lo, hi) if nq else None,
                                       self.vstore.slabs(lo, hi) if nq else None, nq,
                                       np.ascontiguousarray(self.k[lo:hi, nq:]),
                                       np.ascontiguousarray(self.v[lo:hi, nq:]), nr, fmt=self.fmt)
        self._flush_to_rule()
        return out
