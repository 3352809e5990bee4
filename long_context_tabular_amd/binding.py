"""Thin ctypes binding of ``include/sdm_icl_attn.h`` (argument marshalling only).

Every step of the attention path runs in the HIP library; this module only
checks tensor dtypes/devices, passes raw pointers and the current HIP stream,
and turns non-OK status codes into exceptions.  There is no fallback: if
``libsdm_icl_attn.so`` is missing the first call raises.

Function names mirror the C ABI.  PyTorch is used for device memory and
streams only.
"""
from __future__ import annotations

import contextlib
import contextvars
import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdm_icl_attn.so")

SDM_ICL_OK = 0
STATUS_NAMES = {0: "OK", 1: "E_INVALID", 2: "E_UNSUPPORTED", 3: "E_DEVICE", 4: "E_OOM",
                5: "E_HIP", 6: "E_STATE"}
SDM_ICL_SCALE_NONE, SDM_ICL_SCALE_LOG, SDM_ICL_SCALE_GATED_LOG = 0, 1, 2
SDM_ICL_PREC_FP16, SDM_ICL_PREC_FP8_E4M3, SDM_ICL_PREC_AUTO, SDM_ICL_PREC_SCOPED = 0, 1, 2, 3
SDM_ICL_SCOPE_DISABLE, SDM_ICL_SCOPE_ENABLE, SDM_ICL_SCOPE_INHERIT = 0, 1, 2


class SdmIclError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class FitArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("rows_padded", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("lengths", ctypes.POINTER(ctypes.c_int64)),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("head_coef", ctypes.POINTER(ctypes.c_float)),
                ("scale_mode", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("out_ctx", ctypes.c_void_p), ("stream", ctypes.c_void_p)]


class CacheInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("kv_splits", ctypes.c_int32), ("n_valid", ctypes.c_int64),
                ("rows_alloc", ctypes.c_int64), ("keys_per_split", ctypes.c_int64),
                ("length_scalar", ctypes.c_float), ("device_bytes", ctypes.c_uint64),
                ("offloaded", ctypes.c_int32), ("stream_chunk_splits", ctypes.c_int32)]


class ImportArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("lengths", ctypes.POINTER(ctypes.c_int64)), ("scale_mode", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("head_coef", ctypes.POINTER(ctypes.c_float)),
                ("host_k", ctypes.c_void_p), ("host_v", ctypes.c_void_p),
                ("host_scales", ctypes.POINTER(ctypes.c_float)), ("stream", ctypes.c_void_p)]


# name -> (restype, argtypes), exactly the declarations of include/sdm_icl_attn.h
_SIGNATURES = {
    "sdm_icl_attn_fit": (ctypes.c_int32, [ctypes.POINTER(FitArgs), ctypes.POINTER(ctypes.c_void_p)]),
    "sdm_icl_attn_query_workspace_size": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64,
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "sdm_icl_attn_query": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "sdm_icl_attn_query_noalloc": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "sdm_icl_attn_cache_info": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(CacheInfo)]),
    "sdm_icl_attn_cache_export": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p]),
    "sdm_icl_attn_cache_lengths": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                                    ctypes.POINTER(ctypes.c_float)]),
    "sdm_icl_attn_cache_import": (ctypes.c_int32, [ctypes.POINTER(ImportArgs), ctypes.POINTER(ctypes.c_void_p)]),
    "sdm_icl_attn_cache_offload": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sdm_icl_attn_cache_restore": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p]),
    "sdm_icl_attn_release": (ctypes.c_int32, [ctypes.c_void_p]),
    "sdm_icl_log_scale": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.POINTER(ctypes.c_float),
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "sdm_icl_qkv_project": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "sdm_icl_timing_enable": (ctypes.c_int32, [ctypes.c_int32]),
    "sdm_icl_timing_read": (ctypes.c_int32, [ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_int64)]),
    "sdm_icl_length_scalar": (ctypes.c_float, [ctypes.c_int64]),
    "sdm_icl_head_factors": (ctypes.c_int32, [ctypes.c_int64, ctypes.POINTER(ctypes.c_float),
                                              ctypes.c_int32, ctypes.POINTER(ctypes.c_uint16)]),
    "sdm_icl_select_precision": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32]),
    "sdm_icl_split_plan": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "sdm_icl_scope_push": (ctypes.c_int32, [ctypes.c_int32]),
    "sdm_icl_scope_pop": (ctypes.c_int32, []),
    "sdm_icl_scope_fp8": (ctypes.c_int32, []),
    "sdm_icl_last_error": (ctypes.c_char_p, []),
    "sdm_icl_version": (ctypes.c_int32, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_tabular_amd.build_lib` (or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != SDM_ICL_OK:
        raise SdmIclError(status, lib().sdm_icl_last_error().decode())


# The FP8 scope of the Python caller, context-local (threads and asyncio tasks
# each see their own), as the settings of the pages' optimize scope are.  The
# library keeps its scope per OS thread, so every call that depends on it
# pushes this context's effective setting around the C call.
_SCOPE: contextvars.ContextVar = contextvars.ContextVar("sdm_icl_fp8_scope", default=())


def _effective_scope() -> int:
    for setting in reversed(_SCOPE.get()):
        if setting != SDM_ICL_SCOPE_INHERIT:
            return setting
    return SDM_ICL_SCOPE_DISABLE


@contextlib.contextmanager
def optimize(attention: Optional[str] = "fp8"):
    """Opt-in FP8 attention scope: ``attention="fp8"`` enables FP8 for
    intermediate layers (fits with ``SDM_ICL_PREC_SCOPED``), ``"none"``
    disables it, ``None`` inherits the enclosing setting.  Leaving the scope
    restores the previous setting and leaves caches untouched."""
    setting = {"fp8": SDM_ICL_SCOPE_ENABLE, "none": SDM_ICL_SCOPE_DISABLE,
               None: SDM_ICL_SCOPE_INHERIT}.get(attention)
    if setting is None and attention is not None:
        raise ValueError(f"unknown attention optimisation {attention!r}")
    token = _SCOPE.set(_SCOPE.get() + (setting,))
    try:
        yield
    finally:
        _SCOPE.reset(token)


def fp8_scope_enabled() -> bool:
    return _effective_scope() == SDM_ICL_SCOPE_ENABLE


@contextlib.contextmanager
def _c_scope():
    _check(lib().sdm_icl_scope_push(_effective_scope()))
    try:
        yield
    finally:
        _check(lib().sdm_icl_scope_pop())


def _stream_ptr(stream) -> Optional[int]:
    """The HIP stream handle to pass: the given torch stream, else the current
    stream of the current device (read through torch's raw accessor when it
    exists: the public call builds a Stream object, ~3 us per query)."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device()) or None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def _dev_ptr(t, name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# ------------------------------------------------------------------ host helpers

def sdm_icl_version() -> int:
    return lib().sdm_icl_version()


def sdm_icl_last_error() -> str:
    return lib().sdm_icl_last_error().decode()


def sdm_icl_length_scalar(n: int) -> np.float32:
    return np.float32(lib().sdm_icl_length_scalar(int(n)))


def sdm_icl_head_factors(n: int, head_coef) -> np.ndarray:
    coef = np.ascontiguousarray(head_coef, dtype=np.float32)
    out = np.zeros(coef.size, dtype=np.uint16)
    _check(lib().sdm_icl_head_factors(int(n), coef.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                      coef.size, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))))
    return out.view(np.float16)


def sdm_icl_scope_push(setting: int) -> None:
    _check(lib().sdm_icl_scope_push(int(setting)))


def sdm_icl_scope_pop() -> None:
    _check(lib().sdm_icl_scope_pop())


def sdm_icl_scope_fp8() -> int:
    return lib().sdm_icl_scope_fp8()


def sdm_icl_select_precision(n: int, requested: int) -> int:
    return lib().sdm_icl_select_precision(int(n), int(requested))


def sdm_icl_split_plan(n: int, num_cus: int, bh_count: int):
    s = ctypes.c_int32()
    k = ctypes.c_int64()
    _check(lib().sdm_icl_split_plan(int(n), int(num_cus), int(bh_count), ctypes.byref(s),
                                    ctypes.byref(k)))
    return s.value, k.value


SDM_ICL_NOALLOC_SCRATCH_BYTES = 64 << 20
SDM_ICL_TIMING_CONTEXT, SDM_ICL_TIMING_QUERY, SDM_ICL_TIMING_COMBINE = 0, 1, 2
SDM_ICL_TIMING_SCALE, SDM_ICL_TIMING_PREP, SDM_ICL_TIMING_PROJECT = 3, 4, 5


def sdm_icl_timing_enable(on: bool) -> None:
    _check(lib().sdm_icl_timing_enable(1 if on else 0))


def sdm_icl_timing_read(kernel_class: int):
    """(summed milliseconds, launches) of one kernel class since the last read."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().sdm_icl_timing_read(int(kernel_class), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ------------------------------------------------------------------ cache handle

class Cache:
    """Owns one ``sdm_icl_cache`` handle; ``release()`` frees it."""

    def __init__(self, handle: int):
        self.handle = handle

    def info(self) -> dict:
        return sdm_icl_attn_cache_info(self)

    def release(self) -> None:
        if self.handle:
            h, self.handle = self.handle, None
            _check(lib().sdm_icl_attn_release(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.release()


def sdm_icl_attn_fit(q, k, v, length, scale_mode: int = SDM_ICL_SCALE_NONE,
                     precision: int = SDM_ICL_PREC_AUTO, head_coef=None, gate=None,
                     out_ctx=None, stream=None) -> Cache:
    """Build the K/V cache from context q/k/v ``[B, N_pad, H, 64]`` (fp16) with
    ``length`` valid rows (one int for every batch element, or a sequence of
    B ints); if ``out_ctx`` (same shape) is given, the context self-attention
    is written there too."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, N_pad, H, D]")
    B, N, H, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, N, H, D):
            raise ValueError(f"{name} must have the shape of q")
    if gate is not None and tuple(gate.shape) != (B, N, H):
        raise ValueError("gate must be [B, N_pad, H]")
    if out_ctx is not None and tuple(out_ctx.shape) != (B, N, H, D):
        raise ValueError("out_ctx must have the shape of q")
    ls = [int(x) for x in np.asarray(length, dtype=np.int64).reshape(-1)]
    if len(ls) == 1:
        ls = ls * B
    if len(ls) != B:
        raise ValueError("length must be one int or one per batch element")
    lengths = (ctypes.c_int64 * B)(*ls)
    coef = None
    if head_coef is not None:
        coef_np = np.ascontiguousarray(head_coef, dtype=np.float32)
        coef = coef_np.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    f16 = torch.float16
    args = FitArgs(batch=B, rows_padded=N, heads=H, head_dim=D, lengths=lengths,
                   q=_dev_ptr(q, "q", f16), k=_dev_ptr(k, "k", f16), v=_dev_ptr(v, "v", f16),
                   gate=_dev_ptr(gate, "gate", f16), head_coef=coef, scale_mode=scale_mode,
                   precision=precision, out_ctx=_dev_ptr(out_ctx, "out_ctx", f16),
                   stream=_stream_ptr(stream))
    handle = ctypes.c_void_p()
    with _c_scope():
        _check(lib().sdm_icl_attn_fit(ctypes.byref(args), ctypes.byref(handle)))
    return Cache(handle.value)


def sdm_icl_attn_query_workspace_size(cache: Cache, n_query: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().sdm_icl_attn_query_workspace_size(cache.handle, int(n_query), ctypes.byref(b)))
    return b.value


def sdm_icl_attn_query(cache: Cache, q, gate=None, out=None, workspace=None, stream=None):
    """Query rows q ``[B, R, H, 64]`` attend to the cache; returns ``out``."""
    import torch
    B, R, H, D = q.shape
    if gate is not None and tuple(gate.shape) != (B, R, H):
        raise ValueError("gate must be [B, R, H]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != (B, R, H, D):
        raise ValueError("out must have the shape of q")
    if workspace is None:
        need = sdm_icl_attn_query_workspace_size(cache, R)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    with _c_scope():
        _check(lib().sdm_icl_attn_query(cache.handle, _dev_ptr(q, "q", torch.float16),
                                        _dev_ptr(gate, "gate", torch.float16), R,
                                        _dev_ptr(out, "out", torch.float16),
                                        _dev_ptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream)))
    return out


def sdm_icl_attn_query_noalloc(cache: Cache, q, gate=None, out=None, stream=None):
    """sdm_icl_attn_query on the library's per-device scratch array (no
    workspace argument, no device allocation inside the call); returns ``out``."""
    import torch
    B, R, H, D = q.shape
    if gate is not None and tuple(gate.shape) != (B, R, H):
        raise ValueError("gate must be [B, R, H]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != (B, R, H, D):
        raise ValueError("out must have the shape of q")
    with _c_scope():
        _check(lib().sdm_icl_attn_query_noalloc(cache.handle, _dev_ptr(q, "q", torch.float16),
                                                _dev_ptr(gate, "gate", torch.float16), R,
                                                _dev_ptr(out, "out", torch.float16), _stream_ptr(stream)))
    return out


def sdm_icl_attn_cache_info(cache: Cache) -> dict:
    info = CacheInfo()
    _check(lib().sdm_icl_attn_cache_info(cache.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in CacheInfo._fields_}


def sdm_icl_attn_cache_export(cache: Cache, stream=None):
    """(K ``[B,H,n,D]``, V ``[B,H,n,D]``, scales ``[3,B,H]``) on the host:
    uint8 e4m3 codes in FP8 mode, float16 in FP16 mode."""
    i = sdm_icl_attn_cache_info(cache)
    dt = np.uint8 if i["precision"] == SDM_ICL_PREC_FP8_E4M3 else np.float16
    shape = (i["batch"], i["heads"], i["n_valid"], i["head_dim"])
    k = np.empty(shape, dtype=dt)
    v = np.empty(shape, dtype=dt)
    sc = np.empty((3, i["batch"], i["heads"]), dtype=np.float32)
    with _c_scope():
        _check(lib().sdm_icl_attn_cache_export(cache.handle, k.ctypes.data, v.ctypes.data,
                                               sc.ctypes.data, _stream_ptr(stream)))
    return k, v, sc


def sdm_icl_attn_cache_lengths(cache: Cache):
    """(n_b int64 ``[B]``, L32(n_b) float32 ``[B]``) of a cache."""
    B = sdm_icl_attn_cache_info(cache)["batch"]
    n = np.empty(B, dtype=np.int64)
    L = np.empty(B, dtype=np.float32)
    _check(lib().sdm_icl_attn_cache_lengths(cache.handle, n.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                            L.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return n, L


def import_args(k: np.ndarray, v: np.ndarray, scales: np.ndarray, lengths, scale_mode: int,
                precision: int, head_coef=None, stream=None):
    """(ImportArgs, keep-alive tuple) for host arrays as cache_export returns them."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    Bn, H, n, D = k.shape
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    ls = [int(x) for x in np.asarray(lengths, dtype=np.int64).reshape(-1)]
    if len(ls) == 1:
        ls = ls * Bn
    la = (ctypes.c_int64 * Bn)(*ls)
    coef = None
    coef_np = None
    if head_coef is not None:
        coef_np = np.ascontiguousarray(head_coef, dtype=np.float32)
        coef = coef_np.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    args = ImportArgs(batch=Bn, heads=H, head_dim=D, lengths=la, scale_mode=scale_mode,
                      precision=precision, head_coef=coef, host_k=k.ctypes.data, host_v=v.ctypes.data,
                      host_scales=sc.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                      stream=stream)
    return args, (k, v, sc, la, coef_np)


def sdm_icl_attn_cache_import(k: np.ndarray, v: np.ndarray, scales: np.ndarray, lengths,
                              scale_mode: int, precision: int, head_coef=None, stream=None) -> Cache:
    """Rebuild a cache from ``cache_export``'s arrays (K, V ``[B, H, n, 64]``,
    scales ``[3, B, H]``)."""
    args, keep = import_args(k, v, scales, lengths, scale_mode, precision, head_coef, _stream_ptr(stream))
    handle = ctypes.c_void_p()
    _check(lib().sdm_icl_attn_cache_import(ctypes.byref(args), ctypes.byref(handle)))
    return Cache(handle.value)


def sdm_icl_attn_cache_offload(cache: Cache, chunk_bytes: int = 0, stream=None) -> None:
    """Move the cache's K/V to pinned host memory; queries then stream it in
    chunks of at most ``chunk_bytes`` of K (0: the library's default)."""
    _check(lib().sdm_icl_attn_cache_offload(cache.handle, int(chunk_bytes), _stream_ptr(stream)))


def sdm_icl_attn_cache_restore(cache: Cache, stream=None) -> None:
    """Move an offloaded cache's K/V back into device memory."""
    _check(lib().sdm_icl_attn_cache_restore(cache.handle, _stream_ptr(stream)))


def sdm_icl_attn_release(cache: Cache) -> None:
    cache.release()


def sdm_icl_log_scale(q, key_length: int, head_coef=None, scale_mode: int = SDM_ICL_SCALE_LOG,
                      gate=None, q_inv_scale=None, out=None, stream=None):
    """Fused shared-length scaling of q ``[B, rows, H, 64]``; returns the
    head-major ``[B, H, rows, 64]`` fp16 rows, or e4m3 codes (uint8) when
    ``q_inv_scale`` (device float32 ``[B, H]``) is given."""
    import torch
    B, R, H, D = q.shape
    if out is None:
        dtype = torch.uint8 if q_inv_scale is not None else torch.float16
        out = torch.empty((B, H, R, D), dtype=dtype, device=q.device)
    coef = None
    if head_coef is not None:
        coef_np = np.ascontiguousarray(head_coef, dtype=np.float32)
        coef = coef_np.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    _check(lib().sdm_icl_log_scale(_dev_ptr(q, "q", torch.float16), _dev_ptr(gate, "gate", torch.float16),
                                   B, R, H, D, int(key_length), coef, scale_mode,
                                   _dev_ptr(q_inv_scale, "q_inv_scale", torch.float32),
                                   _dev_ptr(out, "out"), _stream_ptr(stream)))
    return out


def sdm_icl_qkv_project(x, w, bias=None, heads: int = 8, key_length: int = 0, head_coef=None,
                        scale_mode: int = SDM_ICL_SCALE_NONE, gate=None, outs=None, stream=None):
    """(q~, k, v) ``[B, rows, H, 64]`` fp16 of hidden rows x ``[B, rows, E]`` and a
    linear layer's weight w ``[3 H 64, E]`` (Q rows, then K, then V), bias
    ``[3 H 64]`` or None; q~ carries ``scale_mode``'s scaling."""
    import torch
    B, R, E = x.shape
    D = 64
    if tuple(w.shape) != (3 * heads * D, E):
        raise ValueError("w must be [3 * heads * 64, in_features]")
    if bias is not None and tuple(bias.shape) != (3 * heads * D,):
        raise ValueError("bias must be [3 * heads * 64]")
    if gate is not None and tuple(gate.shape) != (B, R, heads):
        raise ValueError("gate must be [B, rows, heads]")
    if outs is None:
        outs = tuple(torch.empty((B, R, heads, D), dtype=torch.float16, device=x.device) for _ in range(3))
    coef = None
    coef_np = None
    if head_coef is not None:
        coef_np = np.ascontiguousarray(head_coef, dtype=np.float32)
        coef = coef_np.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    f16 = torch.float16
    _check(lib().sdm_icl_qkv_project(_dev_ptr(x, "x", f16), _dev_ptr(w, "w", f16), _dev_ptr(bias, "bias", f16),
                                     B, R, E, heads, D, int(key_length), coef, scale_mode,
                                     _dev_ptr(gate, "gate", f16), *(_dev_ptr(o, "out", f16) for o in outs),
                                     _stream_ptr(stream)))
    return outs
