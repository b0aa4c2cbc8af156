"""Python binding of libattn.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/attn.h``; this module only checks tensor metadata, allocates
outputs and workspaces through torch, and passes raw device pointers and the
current HIP stream. There is no fallback: without the built library every
call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libattn_debug.so")  # the same library with address checks

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_BF16, ATTN_FP32 = 0, 1
OP_FWD, OP_BWD, OP_DECODE = 0, 1, 2

_DTYPES = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_FP32}


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn status {status}: {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("Tq", ctypes.c_int32),
        ("Tkv", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("kv_lens", ctypes.c_void_p),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
    ]


_lib = None

_P = ctypes.POINTER(Params)
_V = ctypes.c_void_p
_SIGS = {
    "attn_validate": (ctypes.c_int, [_P, ctypes.c_int32]),
    "attn_fwd": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V]),
    "attn_bwd_workspace_size": (ctypes.c_size_t, [_P]),
    "attn_bwd": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "attn_bwd_preprocess": (ctypes.c_int, [_P, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "attn_bwd_dkdv": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "attn_bwd_dq": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "attn_bwd_dq_and_preprocess": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "attn_decode_num_splits": (ctypes.c_int32, [_P]),
    "attn_decode_workspace_size": (ctypes.c_size_t, [_P, ctypes.c_int32]),
    "attn_decode": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, ctypes.c_int32, _V, ctypes.c_size_t, _V]),
    "attn_decode_noalloc": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, ctypes.c_int32, _V]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_debug_take": (ctypes.c_int, [ctypes.POINTER(ctypes.c_ulonglong)]),
    "attn_debug_selftest": (ctypes.c_int, [ctypes.c_void_p]),
}
EXPORTS = tuple(_SIGS)


def load_library(path: str):
    """A handle on a built library at `path`, with every entry point's signature set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m forward_backward_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib(path: str = LIB_PATH):
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(path)
    return _lib


def debug_take(handle=None):
    """(accesses outside the registered buffers, first such address) since the
    last call, from a library built with address checks (libattn_debug.so)."""
    out = (ctypes.c_ulonglong * 2)()
    L = handle if handle is not None else lib()
    status = L.attn_debug_take(out)
    if status != ATTN_OK:
        raise AttnError(status, f"{L.attn_status_string(status).decode()}: {L.attn_last_error().decode()}")
    return int(out[0]), int(out[1])


def _check(status: int):
    if status != ATTN_OK:
        L = lib()
        raise AttnError(status, f"{L.attn_status_string(status).decode()}: {L.attn_last_error().decode()}")


def make_params(B, Tq, Tkv, Hq, Hkv, D, dtype=ATTN_BF16, scale=None, causal=False, kv_lens_ptr=None,
                window=None) -> Params:
    """``window``: ``(left, right)`` local window bounds, negative = none; None = no window."""
    left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    return Params(B, Tq, Tkv, Hq, Hkv, D, dtype, float(1.0 / math.sqrt(D) if scale is None else scale),
                  int(bool(causal)), kv_lens_ptr, left, right)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _tensor4(name, t):
    if not isinstance(t, torch.Tensor) or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D tensor [B, T, H, D]")
    if not _on_device(t):
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be bfloat16 or float32")


def _like(name, t, shape, dtype, device):
    """``t`` must be a contiguous tensor of exactly this shape and dtype on
    ``device``: every pointer handed to the library covers what the kernels
    read or write."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not _on_device(t) or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(ws, need, device):
    """A caller's workspace: contiguous device memory of at least ``need`` bytes.
    Returns its size in bytes."""
    if not isinstance(ws, torch.Tensor):
        raise ValueError("workspace must be a tensor")
    if not _on_device(ws) or ws.device != device:
        raise ValueError(f"workspace must be on {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} needed")
    return nbytes


def _params_for(q, k, scale, causal, kv_lens, window=None):
    _tensor4("q", q)
    _tensor4("k", k)
    if q.dtype != k.dtype:
        raise ValueError("q and k must share a dtype")
    if k.device != q.device:
        raise ValueError("q and k must be on the same GPU")
    if kv_lens is not None:
        _like("kv_lens", kv_lens, (q.shape[0],), torch.int32, q.device)
    B, Tq, Hq, D = q.shape
    _, Tkv, Hkv, _ = k.shape
    return make_params(B, Tq, Tkv, Hq, Hkv, D, _DTYPES[q.dtype], scale, causal,
                       None if kv_lens is None else kv_lens.data_ptr(), window)


def _lse_shape(p):
    return (p.B, p.Hq, p.Tq)


def fwd(q, k, v, scale=None, causal=False, kv_lens=None, out=None, lse=None, window=None):
    """O [B,Tq,Hq,D] (dtype of q) and LSE fp32 [B,Hq,Tq] via attn_fwd."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _like("v", v, k.shape, k.dtype, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty(_lse_shape(p), dtype=torch.float32, device=q.device) if lse is None else lse
    _like("out", o, q.shape, q.dtype, q.device)
    _like("lse", lse_t, _lse_shape(p), torch.float32, q.device)
    _check(lib().attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), _stream()))
    return o, lse_t


def _bwd_inputs(p, q, k, v=None, o=None, lse=None, do=None):
    if v is not None:
        _like("v", v, k.shape, k.dtype, q.device)
    if o is not None:
        _like("o", o, q.shape, q.dtype, q.device)
    if lse is not None:
        _like("lse", lse, _lse_shape(p), torch.float32, q.device)
    if do is not None:
        _like("do", do, q.shape, q.dtype, q.device)


def bwd(q, k, v, o, lse, do, scale=None, causal=False, kv_lens=None, workspace=None, window=None):
    """dQ, dK, dV via attn_bwd (deterministic two-pass backward)."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _bwd_inputs(p, q, k, v, o, lse, do)
    need = lib().attn_bwd_workspace_size(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = _workspace(ws, need, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    _check(lib().attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(ws), nbytes, _stream()))
    return dq, dk, dv


def bwd_workspace(q, k, causal=False, kv_lens=None, window=None):
    """A device workspace large enough for the backward of this problem."""
    p = _params_for(q, k, None, causal, kv_lens, window)
    need = lib().attn_bwd_workspace_size(ctypes.byref(p))
    return torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)


def bwd_preprocess(o, lse, do, ws, q, k, scale=None, causal=False, kv_lens=None, window=None):
    """Pass 1 of the backward: D = rowsum(dO * O), LSE * log2(e) and the row terms into the workspace."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _bwd_inputs(p, q, k, o=o, lse=lse, do=do)
    nbytes = _workspace(ws, lib().attn_bwd_workspace_size(ctypes.byref(p)), q.device)
    _check(lib().attn_bwd_preprocess(ctypes.byref(p), _ptr(o), _ptr(lse), _ptr(do), _ptr(ws), nbytes, _stream()))


def bwd_dkdv(q, k, v, lse, do, ws, dk, dv, scale=None, causal=False, kv_lens=None, window=None):
    """Pass 2 of the backward: dK and dV (needs the preprocess pass, or bwd_dq_and_preprocess, done)."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _bwd_inputs(p, q, k, v=v, lse=lse, do=do)
    _like("dk", dk, k.shape, k.dtype, q.device)
    _like("dv", dv, k.shape, k.dtype, q.device)
    nbytes = _workspace(ws, lib().attn_bwd_workspace_size(ctypes.byref(p)), q.device)
    _check(lib().attn_bwd_dkdv(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dk), _ptr(dv),
                               _ptr(ws), nbytes, _stream()))


def bwd_dq(q, k, v, lse, do, ws, dq, scale=None, causal=False, kv_lens=None, window=None):
    """Pass 3 of the backward: dQ (needs the preprocess pass done)."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _bwd_inputs(p, q, k, v=v, lse=lse, do=do)
    _like("dq", dq, q.shape, q.dtype, q.device)
    nbytes = _workspace(ws, lib().attn_bwd_workspace_size(ctypes.byref(p)), q.device)
    _check(lib().attn_bwd_dq(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dq), _ptr(ws),
                             nbytes, _stream()))


def bwd_dq_and_preprocess(q, k, v, o, lse, do, ws, dq, scale=None, causal=False, kv_lens=None, window=None):
    """dQ and the preprocess pass's workspace contents in one call (one launch at
    bf16 head_dim 64/128); bwd_dkdv may follow it directly."""
    p = _params_for(q, k, scale, causal, kv_lens, window)
    _bwd_inputs(p, q, k, v=v, o=o, lse=lse, do=do)
    _like("dq", dq, q.shape, q.dtype, q.device)
    nbytes = _workspace(ws, lib().attn_bwd_workspace_size(ctypes.byref(p)), q.device)
    _check(lib().attn_bwd_dq_and_preprocess(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                            _ptr(dq), _ptr(ws), nbytes, _stream()))


def decode_workspace(q, k_cache, num_splits=0):
    """A device workspace for attn_decode on this problem, reusable by later
    calls of the same or a smaller problem (not by overlapping calls)."""
    p = _params_for(q, k_cache, None, False, None)
    need = lib().attn_decode_workspace_size(ctypes.byref(p), num_splits)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)


def decode(q, k_cache, v_cache, kv_lens=None, scale=None, num_splits=0, want_lse=True, workspace=None):
    """Split-KV decode: O [B,Tq,Hq,D] bf16 and LSE fp32 [B,Hq,Tq] (or None).
    ``workspace``: one from decode_workspace; without it one is allocated
    for the call."""
    p = _params_for(q, k_cache, scale, False, kv_lens)
    _like("v_cache", v_cache, k_cache.shape, k_cache.dtype, q.device)
    o = torch.empty_like(q)
    lse_t = torch.empty(_lse_shape(p), dtype=torch.float32, device=q.device) if want_lse else None
    need = lib().attn_decode_workspace_size(ctypes.byref(p), num_splits)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = _workspace(ws, need, q.device)
    _check(lib().attn_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse_t),
                             num_splits, _ptr(ws), nbytes, _stream()))
    return o, lse_t


def decode_noalloc(q, k_cache, v_cache, kv_lens=None, scale=None, num_splits=0, out=None, lse=None,
                   want_lse=True):
    """Split-KV decode through attn_decode_noalloc: the library's static
    scratch replaces the workspace, so with ``out`` (and ``lse``) given the
    call allocates nothing."""
    p = _params_for(q, k_cache, scale, False, kv_lens)
    _like("v_cache", v_cache, k_cache.shape, k_cache.dtype, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = lse if lse is not None else (torch.empty(_lse_shape(p), dtype=torch.float32, device=q.device)
                                         if want_lse else None)
    _like("out", o, q.shape, q.dtype, q.device)
    if lse_t is not None:
        _like("lse", lse_t, _lse_shape(p), torch.float32, q.device)
    _check(lib().attn_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse_t),
                                     num_splits, _stream()))
    return o, lse_t


def decode_num_splits(B, Tq, Tkv, Hq, Hkv, D) -> int:
    p = make_params(B, Tq, Tkv, Hq, Hkv, D)
    return int(lib().attn_decode_num_splits(ctypes.byref(p)))
