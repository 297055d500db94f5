"""Python binding of libkivi (argument marshalling only).

Every call checks torch-level properties (dtype, device, strides), builds
the C structs and calls the function of the same name in ``libkivi.so`` on
torch's current HIP stream.  All arithmetic happens in the HIP kernels; if
the library is missing this module raises instead of computing anything.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkivi.so")

KIVI_KEYS = 0
KIVI_VALUES = 1
KIVI_META_F32 = 0
KIVI_META_F16 = 1
KIVI_ATTEND_BF16 = 1
KIVI_ATTEND_VARLEN = 2
HEAD_DIM = 128
GROUP = 32

# symbols of include/kivi.h, include/kivi_cache.h and include/kivi_calib.h
EXPORTS = (
    "kivi_quantize_keys", "kivi_quantize_values", "kivi_dequantize",
    "kivi_quantize_keys_bf16", "kivi_quantize_values_bf16", "kivi_dequantize_bf16",
    "kivi_decode_attend", "kivi_decode_attend_varlen", "kivi_decode_attend_workspace_bytes",
    "kivi_decode_attend_bf16", "kivi_decode_attend_varlen_bf16", "kivi_decode_attend_noalloc",
    "kivi_status_string", "kivi_last_hip_error", "kivi_calib_copy", "kivi_calib_read",
    "kivi_calib_write", "kivi_calib_mix",
    "kivi_cache_device_bytes", "kivi_cache_init", "kivi_cache_prefill", "kivi_cache_append",
    "kivi_cache_attend", "kivi_cache_attend_workspace_bytes", "kivi_cache_end_step",
    "kivi_cache_append_attend",
)
CACHE_MAX_LAYERS = 256


class KiviError(RuntimeError):
    """A libkivi call returned a negative status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class CStore(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("zero", ctypes.c_void_p),
        ("codes_bh_stride", ctypes.c_int64),
        ("meta_bh_stride", ctypes.c_int64),
        ("cap", ctypes.c_int64),
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("meta_format", ctypes.c_int32),
    ]


class CCacheConfig(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("residual_length", ctypes.c_int32), ("flush_tokens", ctypes.c_int32),
        ("store_capacity", ctypes.c_int64), ("meta_format", ctypes.c_int32),
        ("bf16", ctypes.c_int32),
    ]


class CCache(ctypes.Structure):
    _fields_ = [
        ("cfg", CCacheConfig), ("k_store", CStore), ("v_store", CStore),
        ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p), ("k_stage", ctypes.c_void_p),
        ("v_stage", ctypes.c_void_p), ("ring", ctypes.c_int64),
        ("length", ctypes.c_int64), ("n_quant", ctypes.c_int64), ("n_res", ctypes.c_int64),
        ("head", ctypes.c_int64), ("appended", ctypes.c_uint64 * (CACHE_MAX_LAYERS // 64)),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkivi.so (built by ``__graft_entry__.build()``); never falls back."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        sp = ctypes.POINTER(CStore)
        L.kivi_quantize_keys.argtypes = [vp, i64, i64, i64, sp, i64, vp, i64, vp]
        L.kivi_quantize_values.argtypes = [vp, i64, i64, i64, sp, i64, vp, i64, vp]
        L.kivi_dequantize.argtypes = [sp, i64, i64, i64, vp, i64, vp]
        L.kivi_quantize_keys_bf16.argtypes = L.kivi_quantize_keys.argtypes
        L.kivi_quantize_values_bf16.argtypes = L.kivi_quantize_values.argtypes
        L.kivi_dequantize_bf16.argtypes = L.kivi_dequantize.argtypes
        L.kivi_decode_attend.argtypes = [vp, i64, i32, i32, sp, sp, i64, vp, vp, i64, i64,
                                         ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.kivi_decode_attend_varlen.argtypes = [vp, i64, i32, i32, sp, sp, vp, i64, vp, vp, i64,
                                                vp, i64, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.kivi_decode_attend_bf16.argtypes = L.kivi_decode_attend.argtypes
        L.kivi_decode_attend_noalloc.argtypes = [vp, i64, i32, i32, sp, sp, i64, vp, vp, i64, i64,
                                                 ctypes.c_float, vp, vp]
        L.kivi_decode_attend_varlen_bf16.argtypes = L.kivi_decode_attend_varlen.argtypes
        L.kivi_decode_attend_workspace_bytes.argtypes = [i64, i32, i32, i64, i64, i32, i32]
        L.kivi_decode_attend_workspace_bytes.restype = ctypes.c_size_t
        L.kivi_status_string.argtypes = [ctypes.c_int]
        L.kivi_status_string.restype = ctypes.c_char_p
        L.kivi_last_hip_error.argtypes = []
        L.kivi_calib_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.kivi_calib_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.kivi_calib_write.argtypes = [vp, ctypes.c_size_t, vp]
        L.kivi_calib_mix.argtypes = [vp, ctypes.c_size_t, vp, vp]
        cp, cfgp = ctypes.POINTER(CCache), ctypes.POINTER(CCacheConfig)
        L.kivi_cache_device_bytes.argtypes = [cfgp]
        L.kivi_cache_device_bytes.restype = ctypes.c_size_t
        L.kivi_cache_init.argtypes = [cp, cfgp, vp, ctypes.c_size_t]
        L.kivi_cache_prefill.argtypes = [cp, vp, vp, i64, i64, vp]
        L.kivi_cache_append.argtypes = [cp, i32, vp, vp, vp]
        L.kivi_cache_attend.argtypes = [cp, i32, vp, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.kivi_cache_append_attend.argtypes = [cp, i32, vp, vp, vp, i32, ctypes.c_float, vp, vp,
                                               ctypes.c_size_t, vp]
        L.kivi_cache_attend_workspace_bytes.argtypes = [cp, i32]
        L.kivi_cache_attend_workspace_bytes.restype = ctypes.c_size_t
        L.kivi_cache_end_step.argtypes = [cp, vp]
        for name in ("kivi_quantize_keys", "kivi_quantize_values", "kivi_dequantize",
                     "kivi_quantize_keys_bf16", "kivi_quantize_values_bf16", "kivi_dequantize_bf16",
                     "kivi_decode_attend", "kivi_decode_attend_varlen", "kivi_last_hip_error",
                     "kivi_decode_attend_bf16", "kivi_decode_attend_varlen_bf16",
                     "kivi_decode_attend_noalloc", "kivi_calib_copy", "kivi_calib_read", "kivi_calib_write", "kivi_calib_mix",
                     "kivi_cache_init", "kivi_cache_prefill", "kivi_cache_append",
                     "kivi_cache_attend", "kivi_cache_end_step", "kivi_cache_append_attend"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kivi_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise KiviError(rc, what)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _need_f16(t: torch.Tensor, name: str, allow_bf16: bool = False, D: int = HEAD_DIM) -> None:
    if t.dtype != torch.float16 and not (allow_bf16 and t.dtype == torch.bfloat16):
        raise TypeError(f"{name} must be float16{' or bfloat16' if allow_bf16 else ''}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dim() != 3 or t.shape[2] != D or t.stride(2) != 1 or t.stride(1) != D:
        raise ValueError(f"{name} must be [BH][S][{D}] with contiguous token rows")


def _need_query(q: torch.Tensor) -> None:
    if q.dtype not in (torch.float16, torch.bfloat16) or not q.is_cuda or q.dim() != 3 \
            or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16 or bfloat16 device tensor [B][Hq][head_dim]")


def _kv_heads(q: torch.Tensor, k_store: "Store", v_store: "Store") -> int:
    """Hkv of an attend call, after checking that q and both stores agree:
    the C ABI reads q, the residual rows and out at the stores' head_dim and
    B * Hkv slabs, so a mismatch here would be an out-of-bounds access."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][head_dim]")
    B, Hq, D = q.shape
    for st, name in ((k_store, "k_store"), (v_store, "v_store")):
        if st.head_dim != D:
            raise ValueError(f"q has head_dim {D} but {name} has {st.head_dim}")
    if k_store.BH != v_store.BH:
        raise ValueError("k_store and v_store must have the same number of slabs")
    if B == 0:
        return 1
    if k_store.BH % B != 0:
        raise ValueError(f"the stores' {k_store.BH} slabs are not B={B} sequences of kv heads")
    return k_store.BH // B


def _need_out(out: torch.Tensor, B: int, Hq: int, D: int) -> None:
    if not (out.dtype == torch.float32 and out.is_cuda and out.is_contiguous()
            and tuple(out.shape) == (B, Hq, D)):
        raise ValueError(f"out must be a contiguous float32 device tensor of shape ({B}, {Hq}, {D})")


def _need_residual(q: torch.Tensor, k_res: torch.Tensor, v_res: torch.Tensor) -> None:
    _need_f16(k_res, "k_res", allow_bf16=True, D=q.shape[2])
    _need_f16(v_res, "v_res", allow_bf16=True, D=q.shape[2])
    if k_res.dtype != q.dtype or v_res.dtype != q.dtype:
        raise TypeError("k_res and v_res must have the dtype of q")
    if k_res.stride(0) != v_res.stride(0):
        raise ValueError("k_res and v_res must share their slab stride")


class Store:
    """A packed store in device memory (layout of include/kivi.h).

    ``codes`` is int32 storage holding the uint32 code words.  ``meta`` is
    the format of scale and zero: "f32" (float32 tensors) or "f16" (float16
    tensors holding binary16, KIVI_META_F16)."""

    def __init__(self, kind: int, BH: int, cap: int, bits: int = 4, device="cuda",
                 codes: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                 zero: torch.Tensor | None = None, group: int = GROUP, head_dim: int = HEAD_DIM,
                 meta: str = "f32"):
        if meta not in ("f32", "f16"):
            raise ValueError("meta must be 'f32' or 'f16'")
        self.kind, self.BH, self.cap, self.bits, self.group = kind, BH, cap, bits, group
        self.head_dim = head_dim
        self.meta = meta
        self.words = head_dim * bits // 32
        shape = (BH, (cap + group - 1) // group, head_dim) if kind == KIVI_KEYS else \
            (BH, cap, (head_dim + group - 1) // group)
        mdt = torch.float32 if meta == "f32" else torch.float16
        self.codes = codes if codes is not None else torch.zeros((BH, cap, self.words),
                                                                 dtype=torch.int32, device=device)
        self.scale = scale if scale is not None else torch.zeros(shape, dtype=mdt, device=device)
        self.zero = zero if zero is not None else torch.zeros(shape, dtype=mdt, device=device)
        if self.scale.dtype != mdt or self.zero.dtype != mdt:
            raise TypeError("scale and zero must be %s for meta=%r" % (mdt, meta))

    def c(self) -> CStore:
        return CStore(self.codes.data_ptr(), self.scale.data_ptr(), self.zero.data_ptr(),
                      self.codes.stride(0), self.scale.stride(0), self.cap, self.bits,
                      self.group, self.head_dim, self.kind,
                      KIVI_META_F16 if self.meta == "f16" else KIVI_META_F32)

    def nbytes(self) -> int:
        return (self.codes.numel() * 4 + self.scale.numel() * self.scale.element_size()
                + self.zero.numel() * self.zero.element_size())


def _flush(fn_name, x: torch.Tensor, store: Store, dst_token: int, recon, stream):
    _need_f16(x, "x", allow_bf16=True, D=store.head_dim)
    if recon is not None:
        _need_f16(recon, "recon", allow_bf16=True, D=store.head_dim)
        if recon.dtype != x.dtype:
            raise TypeError("recon must have the dtype of x")
    if x.dtype == torch.bfloat16:
        fn_name += "_bf16"
    st = store.c()
    rc = getattr(lib(), fn_name)(
        x.data_ptr(), x.shape[0], x.shape[1], x.stride(0), ctypes.byref(st), dst_token,
        recon.data_ptr() if recon is not None else None,
        recon.stride(0) if recon is not None else 0, _stream(stream))
    _check(rc, fn_name)


def quantize_keys(x: torch.Tensor, store: Store, dst_token: int = 0,
                  recon: torch.Tensor | None = None, stream=None) -> None:
    """kivi_quantize_keys: per-channel key flush of x[BH][S][128] into store
    (kivi_quantize_keys_bf16 when x is bfloat16)."""
    _flush("kivi_quantize_keys", x, store, dst_token, recon, stream)


def quantize_values(x: torch.Tensor, store: Store, dst_token: int = 0,
                    recon: torch.Tensor | None = None, stream=None) -> None:
    """kivi_quantize_values: per-token value flush of x[BH][S][128] into store
    (kivi_quantize_values_bf16 when x is bfloat16)."""
    _flush("kivi_quantize_values", x, store, dst_token, recon, stream)


def dequantize(store: Store, token_begin: int, n_tokens: int, out: torch.Tensor | None = None,
               BH: int | None = None, stream=None, dtype=torch.float16) -> torch.Tensor:
    """kivi_dequantize: fp16 [BH][n_tokens][128] reconstruction of a token range
    (kivi_dequantize_bf16 for a bfloat16 ``out`` / ``dtype``)."""
    BH = store.BH if BH is None else BH
    if out is None:
        out = torch.empty((BH, n_tokens, store.head_dim), dtype=dtype, device=store.codes.device)
    _need_f16(out, "out", allow_bf16=True, D=store.head_dim)
    name = "kivi_dequantize_bf16" if out.dtype == torch.bfloat16 else "kivi_dequantize"
    st = store.c()
    rc = getattr(lib(), name)(ctypes.byref(st), BH, token_begin, n_tokens, out.data_ptr(),
                              out.stride(0), _stream(stream))
    _check(rc, name)
    return out


def attend_workspace_bytes(B: int, Hq: int, Hkv: int, n_quant: int, n_res: int,
                           head_dim: int = HEAD_DIM, bf16: bool = False, varlen: bool = False) -> int:
    """kivi_decode_attend_workspace_bytes for the attend call with these
    arguments (the varlen calls: their max_n_quant / max_n_res)."""
    flags = (KIVI_ATTEND_BF16 if bf16 else 0) | (KIVI_ATTEND_VARLEN if varlen else 0)
    return int(lib().kivi_decode_attend_workspace_bytes(B, Hq, Hkv, n_quant, n_res, head_dim, flags))


def attend_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A new attend workspace of nbytes (its contents do not matter)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def decode_attend(q: torch.Tensor, k_store: Store, v_store: Store, n_quant: int,
                  k_res: torch.Tensor | None, v_res: torch.Tensor | None, n_res: int,
                  softmax_scale: float | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kivi_decode_attend: fp32 [B][Hq][128] attention of one query token per
    sequence over store tokens [0, n_quant) then residual tokens [0, n_res)
    (kivi_decode_attend_bf16 when q is bfloat16; the residual then is too)."""
    Hkv = _kv_heads(q, k_store, v_store)
    _need_query(q)
    B, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need_out(out, B, Hq, D)
    if workspace is None:
        need = attend_workspace_bytes(B, Hq, Hkv, n_quant, n_res, D, q.dtype == torch.bfloat16) if B else 0
        workspace = attend_workspace(need, q.device)
    if n_res > 0:
        _need_residual(q, k_res, v_res)
    ks, vs = k_store.c(), v_store.c()
    name = "kivi_decode_attend_bf16" if q.dtype == torch.bfloat16 else "kivi_decode_attend"
    rc = getattr(lib(), name)(
        q.data_ptr(), B, Hq, Hkv, ctypes.byref(ks), ctypes.byref(vs), n_quant,
        k_res.data_ptr() if n_res > 0 else None, v_res.data_ptr() if n_res > 0 else None,
        k_res.stride(0) if n_res > 0 else 0, n_res, float(softmax_scale), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, name)
    return out


def decode_attend_noalloc(q: torch.Tensor, k_store: Store, v_store: Store, n_quant: int,
                          k_res: torch.Tensor | None, v_res: torch.Tensor | None, n_res: int,
                          softmax_scale: float | None = None, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """kivi_decode_attend_noalloc: decode_attend with the library's own
    device array as workspace (fp16 caches).  Allocates nothing itself when
    ``out`` is given."""
    Hkv = _kv_heads(q, k_store, v_store)
    _need_query(q)
    if q.dtype != torch.float16:
        raise TypeError("kivi_decode_attend_noalloc takes float16 caches")
    B, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need_out(out, B, Hq, D)
    if n_res > 0:
        _need_residual(q, k_res, v_res)
    ks, vs = k_store.c(), v_store.c()
    rc = lib().kivi_decode_attend_noalloc(
        q.data_ptr(), B, Hq, Hkv, ctypes.byref(ks), ctypes.byref(vs), n_quant,
        k_res.data_ptr() if n_res > 0 else None, v_res.data_ptr() if n_res > 0 else None,
        k_res.stride(0) if n_res > 0 else 0, n_res, float(softmax_scale), out.data_ptr(),
        _stream(stream))
    _check(rc, "kivi_decode_attend_noalloc")
    return out


def decode_attend_varlen(q: torch.Tensor, k_store: Store, v_store: Store, n_quant: torch.Tensor,
                         max_n_quant: int, k_res: torch.Tensor | None, v_res: torch.Tensor | None,
                         n_res: torch.Tensor, max_n_res: int, softmax_scale: float | None = None,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """kivi_decode_attend_varlen: like decode_attend, with device int32 [B]
    per-sequence lengths n_quant[b] <= max_n_quant and n_res[b] <= max_n_res
    (kivi_decode_attend_varlen_bf16 when q is bfloat16)."""
    Hkv = _kv_heads(q, k_store, v_store)
    _need_query(q)
    B, Hq, D = q.shape
    for t, name in ((n_quant, "n_quant"), (n_res, "n_res")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.numel() != B:
            raise ValueError(f"{name} must be a contiguous int32 device tensor of B elements")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need_out(out, B, Hq, D)
    if workspace is None:
        need = attend_workspace_bytes(B, Hq, Hkv, max_n_quant, max_n_res, D, q.dtype == torch.bfloat16,
                                      varlen=True) if B else 0
        workspace = attend_workspace(need, q.device)
    if max_n_res > 0:
        _need_residual(q, k_res, v_res)
    ks, vs = k_store.c(), v_store.c()
    name = "kivi_decode_attend_varlen_bf16" if q.dtype == torch.bfloat16 else "kivi_decode_attend_varlen"
    rc = getattr(lib(), name)(
        q.data_ptr(), B, Hq, Hkv, ctypes.byref(ks), ctypes.byref(vs), n_quant.data_ptr(), max_n_quant,
        k_res.data_ptr() if max_n_res > 0 else None, v_res.data_ptr() if max_n_res > 0 else None,
        k_res.stride(0) if max_n_res > 0 else 0, n_res.data_ptr(), max_n_res, float(softmax_scale),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(rc, name)
    return out


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def calib_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """kivi_calib_copy: device-to-device streaming copy (bandwidth ceiling)."""
    n = _nbytes(src)
    if _nbytes(dst) < n:
        raise ValueError("dst is smaller than src")
    _check(lib().kivi_calib_copy(src.data_ptr(), dst.data_ptr(), n, _stream(stream)), "kivi_calib_copy")


def calib_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """kivi_calib_read: read every byte of src (read-only ceiling)."""
    if _nbytes(sink) < 16:
        raise ValueError("sink must hold at least 16 bytes")
    _check(lib().kivi_calib_read(src.data_ptr(), _nbytes(src), sink.data_ptr(), _stream(stream)),
           "kivi_calib_read")


def calib_write(dst: torch.Tensor, stream=None) -> None:
    """kivi_calib_write: write every byte of dst (write-only ceiling)."""
    _check(lib().kivi_calib_write(dst.data_ptr(), _nbytes(dst), _stream(stream)), "kivi_calib_write")


def calib_mix(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """kivi_calib_mix: read src, write 3/8 of its size to dst (the 4-bit
    flush's read:write ratio)."""
    n = _nbytes(src)
    if _nbytes(dst) < n * 3 // 8:
        raise ValueError("dst must hold 3/8 of src's bytes")
    _check(lib().kivi_calib_mix(src.data_ptr(), n, dst.data_ptr(), _stream(stream)), "kivi_calib_mix")


class Cache:
    """kivi_cache (include/kivi_cache.h): every layer's stores and fp16
    residual rings in one device buffer, with the per-step calls.  The
    device buffer is a torch uint8 tensor this object owns; all state
    changes happen in the C calls."""

    def __init__(self, layers: int, batch: int, kv_heads: int, store_capacity: int, bits: int = 4,
                 residual_length: int = 128, flush_tokens: int = GROUP, device="cuda",
                 meta: str = "f32", dtype=torch.float16, group: int = GROUP, head_dim: int = HEAD_DIM):
        if meta not in ("f32", "f16"):
            raise ValueError("meta must be 'f32' or 'f16'")
        if dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("dtype must be torch.float16 or torch.bfloat16")
        self.meta, self.dtype = meta, dtype
        self.group, self.head_dim = group, head_dim
        self.cfg = CCacheConfig(layers, batch, kv_heads, bits, head_dim, group, residual_length,
                                flush_tokens, store_capacity,
                                KIVI_META_F16 if meta == "f16" else KIVI_META_F32,
                                1 if dtype == torch.bfloat16 else 0)
        n = int(lib().kivi_cache_device_bytes(ctypes.byref(self.cfg)))
        if n == 0:
            raise KiviError(-3, "kivi_cache_device_bytes")
        self.buffer = torch.empty(n + 256, dtype=torch.uint8, device=device)
        pad = (-self.buffer.data_ptr()) % 256
        self.buffer = self.buffer[pad:pad + n]
        self.c = CCache()
        _check(lib().kivi_cache_init(ctypes.byref(self.c), ctypes.byref(self.cfg),
                                     self.buffer.data_ptr(), n), "kivi_cache_init")
        self.slabs = layers * batch * kv_heads

    # ---- state (read from the C struct)
    length = property(lambda self: self.c.length)
    n_quant = property(lambda self: self.c.n_quant)
    n_res = property(lambda self: self.c.n_res)
    head = property(lambda self: self.c.head)
    ring = property(lambda self: self.c.ring)

    def _view(self, ptr: int, dtype, shape):
        off = ptr - self.buffer.data_ptr()
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + nbytes].view(dtype).view(shape)

    def stores(self) -> tuple[Store, Store]:
        """The key and value stores of all layers (torch views of the buffer)."""
        out = []
        for cs, kind in ((self.c.k_store, KIVI_KEYS), (self.c.v_store, KIVI_VALUES)):
            D, G = self.head_dim, self.group
            cap, words = cs.cap, D * cs.bits // 32
            meta = (self.slabs, cap // G, D) if kind == KIVI_KEYS else \
                (self.slabs, cap, (D + G - 1) // G)
            mdt = torch.float16 if self.meta == "f16" else torch.float32
            out.append(Store(kind, self.slabs, cap, cs.bits, group=G, head_dim=D,
                             codes=self._view(cs.codes, torch.int32, (self.slabs, cap, words)),
                             scale=self._view(cs.scale, mdt, meta),
                             zero=self._view(cs.zero, mdt, meta), meta=self.meta))
        return out[0], out[1]

    def rings(self) -> tuple[torch.Tensor, torch.Tensor]:
        """[slabs][ring][128] residual rings in the cache's dtype (torch views
        of the buffer)."""
        shape = (self.slabs, self.c.ring, self.head_dim)
        return (self._view(self.c.k_ring, self.dtype, shape),
                self._view(self.c.v_ring, self.dtype, shape))

    # ---- calls
    def _need_dtype(self, t: torch.Tensor, name: str) -> None:
        if t.dtype != self.dtype:
            raise TypeError(f"{name} must be {self.dtype} for this cache, got {t.dtype}")

    def prefill(self, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        _need_f16(k, "k", allow_bf16=True, D=self.head_dim)
        _need_f16(v, "v", allow_bf16=True, D=self.head_dim)
        self._need_dtype(k, "k")
        self._need_dtype(v, "v")
        if k.stride(0) != v.stride(0) or k.shape != v.shape:
            raise ValueError("k and v must have one shape and slab stride")
        _check(lib().kivi_cache_prefill(ctypes.byref(self.c), k.data_ptr(), v.data_ptr(), k.stride(0),
                                        k.shape[1], _stream(stream)), "kivi_cache_prefill")

    def append(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            self._need_dtype(t, name)
            if not t.is_cuda or not t.is_contiguous() or \
                    t.numel() != self.cfg.batch * self.cfg.kv_heads * self.head_dim:
                raise ValueError(f"{name} must be a contiguous device tensor [batch*kv_heads][head_dim]")
        _check(lib().kivi_cache_append(ctypes.byref(self.c), layer, k_new.data_ptr(), v_new.data_ptr(),
                                       _stream(stream)), "kivi_cache_append")

    def attend_workspace_bytes(self, Hq: int) -> int:
        return int(lib().kivi_cache_attend_workspace_bytes(ctypes.byref(self.c), Hq))

    def attend(self, layer: int, q: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, softmax_scale: float | None = None,
               stream=None) -> torch.Tensor:
        if q.dim() != 3 or q.shape[0] != self.cfg.batch or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [{self.cfg.batch}][Hq][{self.head_dim}] for this cache, "
                             f"got {tuple(q.shape)}")
        _need_query(q)
        self._need_dtype(q, "q")
        B, Hq, D = q.shape
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(D)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        _need_out(out, B, Hq, D)
        if workspace is None:
            workspace = attend_workspace(self.attend_workspace_bytes(Hq), q.device)
        _check(lib().kivi_cache_attend(ctypes.byref(self.c), layer, q.data_ptr(), Hq, float(softmax_scale),
                                       out.data_ptr(), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
               "kivi_cache_attend")
        return out

    def append_attend(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      softmax_scale: float | None = None, stream=None) -> torch.Tensor:
        """kivi_cache_append_attend: append then attend in one launch pair
        (the same cache state and a bit-identical out)."""
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            self._need_dtype(t, name)
            if not t.is_cuda or not t.is_contiguous() or \
                    t.numel() != self.cfg.batch * self.cfg.kv_heads * self.head_dim:
                raise ValueError(f"{name} must be a contiguous device tensor [batch*kv_heads][head_dim]")
        if q.dim() != 3 or q.shape[0] != self.cfg.batch or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [{self.cfg.batch}][Hq][{self.head_dim}] for this cache, "
                             f"got {tuple(q.shape)}")
        _need_query(q)
        self._need_dtype(q, "q")
        B, Hq, D = q.shape
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(D)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        _need_out(out, B, Hq, D)
        if workspace is None:
            workspace = attend_workspace(self.attend_workspace_bytes(Hq), q.device)
        _check(lib().kivi_cache_append_attend(ctypes.byref(self.c), layer, k_new.data_ptr(), v_new.data_ptr(),
                                              q.data_ptr(), Hq, float(softmax_scale), out.data_ptr(),
                                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                              _stream(stream)), "kivi_cache_append_attend")
        return out

    def end_step(self, stream=None) -> int:
        rc = lib().kivi_cache_end_step(ctypes.byref(self.c), _stream(stream))
        if rc < 0:
            raise KiviError(rc, "kivi_cache_end_step")
        return rc
