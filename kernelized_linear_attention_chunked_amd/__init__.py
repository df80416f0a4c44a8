"""Python binding of liblinattn (kernelized linear attention on MI355X / gfx950).

Thin ctypes layer over the C ABI declared in ``include/liblinattn.h``: it checks
that tensors are CUDA (HIP) tensors of the right dtype and shape, allocates the
outputs and workspace with PyTorch, and passes raw device pointers plus the
current stream.  Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback.  If the shared library is missing
or cannot be loaded, every call raises.

Functions carry the C names:

* :func:`la_initial_state` -- zero streaming state (Keras proposal, "Streaming
  State", get_initial_state).
* :func:`la_forward` -- causal / non-causal attention with masks and streaming
  state (Keras proposal, "Mathematical definition", "Masking").
* :func:`la_step` -- one T=1 causal decode step.
* :func:`la_gated_forward` -- gated / linear recurrence with GQA (the
  LinearAttention operator page, ai.onnx since version 27).
* :func:`la_gated_step` -- one token of that recurrence (decode).
* :func:`la_delta_forward` -- the delta / gated-delta rules of the same operator.
* :func:`la_backward` -- gradients of the causal :func:`la_forward`.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import LIB_PATH, build as _build

__all__ = [
    "LinAttnError", "la_initial_state", "la_forward", "la_step", "la_gated_forward",
    "la_gated_step", "la_delta_forward", "la_backward", "la_workspace_size", "la_gated_workspace_size", "library_path", "load_library",
    "EXPORTED_SYMBOLS",
]

EXPORTED_SYMBOLS = (
    "la_initial_state", "la_workspace_size", "la_forward", "la_step", "la_gated_workspace_size",
    "la_gated_forward", "la_gated_step", "la_delta_forward", "la_backward_workspace_size",
    "la_backward", "la_status_string", "la_last_error_message",
)

_FM = {"elu_plus_one": 0, "relu": 1}
_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

_lock = threading.Lock()
_lib = None


class LinAttnError(RuntimeError):
    """A liblinattn call returned a non-OK status."""

    def __init__(self, status: int, name: str, message: str):
        super().__init__("%s: %s" % (name, message))
        self.status = status
        self.name = name


def library_path() -> str:
    return LIB_PATH


def load_library(build_if_missing: bool = True):
    """Load liblinattn.so from the package directory (building it only if absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise OSError("liblinattn.so is not built: run kernelized_linear_attention_chunked_amd.build")
            _build()
        lib = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                ctypes.c_size_t)
        lib.la_initial_state.argtypes = [p, p, i64, i64, i64, i64, p]
        lib.la_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        lib.la_forward.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, f32, p,
                                   i64, i64, i64, i64, i64, i32, p, sz, p]
        lib.la_step.argtypes = [p, p, p, p, p, p, p, p, i32, i32, f32, p, i64, i64, i64, i64, i32, p]
        lib.la_gated_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32,
                                                ctypes.POINTER(sz)]
        lib.la_gated_forward.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                         f32, p, sz, p]
        lib.la_gated_step.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i32, f32, p]
        lib.la_delta_forward.argtypes = [p, p, p, p, i32, p, i32, p, p, p, i64, i64, i64, i64, i64, i64,
                                         i32, f32, p]
        lib.la_backward_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        lib.la_backward.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, f32, p, p, p, p, p, i64, i64, i64,
                                    i64, i64, i32, p, sz, p]
        for name in ("la_initial_state", "la_workspace_size", "la_forward", "la_step",
                     "la_gated_workspace_size", "la_gated_forward", "la_gated_step",
                     "la_delta_forward", "la_backward_workspace_size", "la_backward"):
            getattr(lib, name).restype = ctypes.c_int
        lib.la_status_string.argtypes = [ctypes.c_int]
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_last_error_message.argtypes = []
        lib.la_last_error_message.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(rc: int, what: str):
    if rc != 0:
        lib = load_library()
        raise LinAttnError(rc, lib.la_status_string(rc).decode(),
                           "%s: %s" % (what, lib.la_last_error_message().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        # any other dtype is handed to the library, which rejects it
        return 99
    return _DT[t.dtype]


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("liblinattn works on GPU tensors only")


def _contig(t):
    return None if t is None else t.contiguous()


def _mask_u8(mask, B, T, device):
    if mask is None:
        return None
    m = torch.as_tensor(mask, device=device)
    return torch.broadcast_to(m.to(torch.bool), (B, T)).to(torch.uint8).contiguous()


def la_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16, causal=True) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().la_workspace_size(B, T, H, Dk, Dv, _DT.get(dtype, 99), int(bool(causal)),
                                            ctypes.byref(n)), "la_workspace_size")
    return n.value


def la_gated_workspace_size(B, T, Hq, Hkv, Dk, Dv, dtype=torch.bfloat16, per_dim_decay=False) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().la_gated_workspace_size(B, T, Hq, Hkv, Dk, Dv, _DT.get(dtype, 99),
                                                  int(bool(per_dim_decay)), ctypes.byref(n)),
           "la_gated_workspace_size")
    return n.value


def la_initial_state(batch_size, num_heads, key_dim, value_dim=None, use_normalizer=True,
                     device="cuda", out=None):
    """Zero state (kv (B,H,Dk,Dv), k (B,H,Dk) or None), float32, on ``device``.

    ``out``: existing (kv, k) buffers to zero instead of allocating new ones."""
    value_dim = key_dim if value_dim is None else value_dim
    lib = load_library()
    if out is not None:
        kv, k = out
    else:
        kv = torch.empty((batch_size, num_heads, key_dim, value_dim), dtype=torch.float32,
                         device=device)
        k = (torch.empty((batch_size, num_heads, key_dim), dtype=torch.float32, device=device)
             if use_normalizer else None)
    _check(lib.la_initial_state(_ptr(kv), _ptr(k), batch_size, num_heads, key_dim, value_dim,
                                _stream(kv.device)), "la_initial_state")
    return (kv, k) if use_normalizer else (kv, None)


def la_forward(q, k, v, mask=None, state=None, causal=True, feature_map="elu_plus_one",
               use_normalizer=True, eps=1e-6, return_state=False, out=None, state_out=None,
               workspace=None):
    """Linear attention over q,k (B,T,H,Dk), v (B,T,H,Dv).

    ``state``: (kv, k) tuple (k None without the normalizer) or None for zeros.
    ``state_out``: optional (kv, k) buffers for the final state (may be ``state``
    itself for in-place streaming).  Returns ``out`` or ``(out, (kv, k))``.
    """
    _need_cuda(q, k, v)
    q, k, v = _contig(q), _contig(k), _contig(v)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype and (B,T,H) with matching Dk")
    dev = q.device
    lib = load_library()
    m = _mask_u8(mask, B, T, dev)
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    s_in_kv, s_in_k = (None, None) if state is None else state
    s_out_kv = s_out_k = None
    if causal and (return_state or state_out is not None):
        if state_out is not None:
            s_out_kv, s_out_k = state_out
        else:
            s_out_kv = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
            s_out_k = (torch.empty((B, H, Dk), dtype=torch.float32, device=dev)
                       if use_normalizer else None)
    ws_bytes = la_workspace_size(B, T, H, Dk, Dv, q.dtype, causal) if q.dtype in _DT else 0
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.la_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_in_kv), _ptr(s_in_k),
                          _ptr(s_out_kv), _ptr(s_out_k), int(bool(causal)), _FM[feature_map],
                          int(bool(use_normalizer)), float(eps), _ptr(out), B, T, H, Dk, Dv,
                          _dtype_code(q), _ptr(workspace),
                          0 if workspace is None else workspace.numel() * workspace.element_size(),
                          _stream(dev)), "la_forward")
    if return_state and causal:
        return out, (s_out_kv, s_out_k)
    return out


def la_step(q, k, v, state, mask=None, feature_map="elu_plus_one", use_normalizer=True, eps=1e-6,
            out=None, state_out=None, in_place=True):
    """One T=1 decode step.  q,k: (B,H,Dk) or (B,1,H,Dk); v likewise.

    Updates ``state`` in place by default (``in_place``); otherwise writes to
    ``state_out`` or fresh buffers.  Returns ``(out (B,H,Dv), (kv, k))``.
    """
    _need_cuda(q, k, v)
    squeeze = q.dim() == 4
    if squeeze:
        q, k, v = q[:, 0], k[:, 0], v[:, 0]
    q, k, v = _contig(q), _contig(k), _contig(v)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    lib = load_library()
    s_kv, s_k = state
    if in_place:
        o_kv, o_k = s_kv, s_k
    elif state_out is not None:
        o_kv, o_k = state_out
    else:
        o_kv = torch.empty_like(s_kv)
        o_k = torch.empty_like(s_k) if s_k is not None else None
    m = None
    if mask is not None:
        m = torch.broadcast_to(torch.as_tensor(mask, device=dev).to(torch.bool).reshape(-1),
                               (B,)).to(torch.uint8).contiguous()
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check(lib.la_step(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_kv), _ptr(s_k), _ptr(o_kv),
                       _ptr(o_k), _FM[feature_map], int(bool(use_normalizer)), float(eps), _ptr(out),
                       B, H, Dk, Dv, _dtype_code(q), _stream(dev)), "la_step")
    return (out[:, None] if squeeze else out), (o_kv, o_k)


def la_gated_forward(query, key, value, q_num_heads, kv_num_heads, decay=None, past_state=None,
                     scale=0.0, out=None, present_state=None, workspace=None):
    """Gated / linear recurrence on packed (B,T,H*D) tensors with GQA.

    ``decay``: log-space, (B,T,Hkv) per kv head or (B,T,Hkv*Dk) per key
    dimension, or None ("linear" rule).
    Returns ``(output (B,T,Hq*Dv), present_state (B,Hkv,Dk,Dv) float32)``.
    """
    _need_cuda(query, key, value, decay, past_state)
    q, k, v, g = _contig(query), _contig(key), _contig(value), _contig(decay)
    B, T, qw = q.shape
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    if Hq < 1 or Hkv < 1 or qw % Hq or key.shape[-1] % Hkv or value.shape[-1] % Hkv:
        raise ValueError("head counts do not divide the packed widths")
    Dk = qw // Hq
    Dv = value.shape[-1] // Hkv
    dev = q.device
    lib = load_library()
    per_dim = g is not None and tuple(g.shape) == (B, T, Hkv * Dk) and Dk > 1
    if g is not None and not per_dim and tuple(g.shape) != (B, T, Hkv):
        raise ValueError("decay must be (B,T,Hkv) (per kv head) or (B,T,Hkv*Dk) (per key dim)")
    if g is not None and g.dtype != q.dtype:
        raise ValueError("decay must have the dtype of the query")
    if out is None:
        out = torch.empty((B, T, Hq * Dv), dtype=q.dtype, device=dev)
    if present_state is None:
        present_state = torch.empty((B, Hkv, Dk, Dv), dtype=torch.float32, device=dev)
    ws_bytes = (la_gated_workspace_size(B, T, Hq, Hkv, Dk, Dv, q.dtype, per_dim)
                if q.dtype in _DT else 0)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.la_gated_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(_contig(past_state)),
                                _ptr(present_state), _ptr(out), B, T, Hq, Hkv, Dk, Dv,
                                _dtype_code(q), float(scale), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(dev)),
           "la_gated_forward")
    return out, present_state


def la_gated_step(query, key, value, q_num_heads, kv_num_heads, decay=None, past_state=None,
                  scale=0.0, out=None, present_state=None, in_place=False):
    """One token of the gated / linear recurrence: query (B,Hq*Dk) or (B,1,Hq*Dk),
    key / value (B,Hkv*D) or (B,1,Hkv*D), decay (B,Hkv) per kv head or
    (B,Hkv*Dk) per key dim (either with an optional token axis of 1), or None.

    ``in_place`` writes the new state over ``past_state``.  Returns
    ``(output, present_state (B,Hkv,Dk,Dv) float32)``, the output shaped like
    the query.
    """
    _need_cuda(query, key, value, decay, past_state)
    squeeze = query.dim() == 3
    q, k, v, g = _contig(query), _contig(key), _contig(value), _contig(decay)
    if squeeze:
        if q.shape[1] != 1 or k.shape[1] != 1 or v.shape[1] != 1:
            raise ValueError("la_gated_step takes one token")
        q, k, v = q[:, 0], k[:, 0], v[:, 0]
        g = None if g is None else g.reshape(g.shape[0], -1)
    B, qw = q.shape
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    if Hq < 1 or Hkv < 1 or qw % Hq or k.shape[-1] % Hkv or v.shape[-1] % Hkv:
        raise ValueError("head counts do not divide the packed widths")
    Dk = qw // Hq
    Dv = v.shape[-1] // Hkv
    dev = q.device
    lib = load_library()
    per_dim = g is not None and tuple(g.shape) == (B, Hkv * Dk) and Dk > 1
    if g is not None and not per_dim and tuple(g.shape) != (B, Hkv):
        raise ValueError("decay must be (B,Hkv) (per kv head) or (B,Hkv*Dk) (per key dim)")
    if g is not None and g.dtype != q.dtype:
        raise ValueError("decay must have the dtype of the query")
    past = _contig(past_state)
    if in_place:
        if past is None:
            raise ValueError("in_place needs past_state")
        present_state = past
    elif present_state is None:
        present_state = torch.empty((B, Hkv, Dk, Dv), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, Hq * Dv), dtype=q.dtype, device=dev)
    _check(lib.la_gated_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(past), _ptr(present_state),
                             _ptr(out), B, Hq, Hkv, Dk, Dv, _dtype_code(q), float(scale), _stream(dev)),
           "la_gated_step")
    return (out[:, None] if squeeze else out), present_state


def la_delta_forward(query, key, value, q_num_heads, kv_num_heads, beta, decay=None, past_state=None,
                     scale=0.0, out=None, present_state=None):
    """Delta rule (``decay`` None) or gated delta rule on packed (B,T,H*D) tensors
    with GQA.  ``beta``: (B,T,Hkv) or (B,T,1); ``decay``: log-space, (B,T,Hkv)
    or (B,T,Hkv*Dk).  Returns ``(output (B,T,Hq*Dv), present_state (B,Hkv,Dk,Dv)
    float32)``.
    """
    _need_cuda(query, key, value, beta, decay, past_state)
    q, k, v, g, be = _contig(query), _contig(key), _contig(value), _contig(decay), _contig(beta)
    B, T, qw = q.shape
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    if Hq < 1 or Hkv < 1 or qw % Hq or k.shape[-1] % Hkv or v.shape[-1] % Hkv:
        raise ValueError("head counts do not divide the packed widths")
    Dk = qw // Hq
    Dv = v.shape[-1] // Hkv
    dev = q.device
    lib = load_library()
    per_dim = g is not None and tuple(g.shape) == (B, T, Hkv * Dk) and Dk > 1
    if g is not None and not per_dim and tuple(g.shape) != (B, T, Hkv):
        raise ValueError("decay must be (B,T,Hkv) (per kv head) or (B,T,Hkv*Dk) (per key dim)")
    if tuple(be.shape) not in ((B, T, Hkv), (B, T, 1)):
        raise ValueError("beta must be (B,T,Hkv) or (B,T,1)")
    beta_per_head = tuple(be.shape) == (B, T, Hkv) and Hkv > 1
    for t in (g, be):
        if t is not None and t.dtype != q.dtype:
            raise ValueError("decay and beta must have the dtype of the query")
    if out is None:
        out = torch.empty((B, T, Hq * Dv), dtype=q.dtype, device=dev)
    if present_state is None:
        present_state = torch.empty((B, Hkv, Dk, Dv), dtype=torch.float32, device=dev)
    _check(lib.la_delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(be),
                                int(beta_per_head), _ptr(_contig(past_state)), _ptr(present_state),
                                _ptr(out), B, T, Hq, Hkv, Dk, Dv, _dtype_code(q), float(scale),
                                _stream(dev)), "la_delta_forward")
    return out, present_state


def la_backward(q, k, v, dout, mask=None, state=None, dstate=None, feature_map="elu_plus_one",
                use_normalizer=True, eps=1e-6):
    """Gradients of the causal ``la_forward(q, k, v, mask, state, ...)`` for the
    loss sum(dout * out) + <dstate, state_out>.

    ``state``: the forward's (kv, k) initial state or None; ``dstate``: (dkv, dk)
    gradient of its final state or None.  Returns ``(dq, dk, dv, (dS0, dZ0))``,
    dZ0 None without the normalizer.
    """
    _need_cuda(q, k, v, dout)
    q, k, v, dout = _contig(q), _contig(k), _contig(v), _contig(dout)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    lib = load_library()
    m = _mask_u8(mask, B, T, dev)
    s_kv, s_k = (None, None) if state is None else state
    g_kv, g_k = (None, None) if dstate is None else dstate
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dS0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    dZ0 = torch.empty((B, H, Dk), dtype=torch.float32, device=dev) if use_normalizer else None
    n = ctypes.c_size_t(0)
    _check(lib.la_backward_workspace_size(B, T, H, Dk, Dv, _dtype_code(q), int(bool(use_normalizer)),
                                          ctypes.byref(n)), "la_backward_workspace_size")
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev)
    _check(lib.la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(_contig(s_kv)), _ptr(_contig(s_k)),
                           _ptr(dout), _ptr(_contig(g_kv)), _ptr(_contig(g_k)), _FM[feature_map],
                           int(bool(use_normalizer)), float(eps), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dS0),
                           _ptr(dZ0), B, T, H, Dk, Dv, _dtype_code(q), _ptr(ws), n.value, _stream(dev)),
           "la_backward")
    return dq, dk, dv, (dS0, dZ0)
