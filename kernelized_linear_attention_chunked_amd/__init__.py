"""Python binding of liblinattn (kernelized linear attention on MI355X / gfx950).

Thin ctypes layer over the C ABI declared in ``include/liblinattn.h``: it checks
that every tensor is a GPU tensor on the inputs' device with the dtype and shape
the call needs, allocates the outputs and workspace with PyTorch, and passes
raw device pointers plus the current stream.  Inputs that are not contiguous
are copied, and each copy is held until the library has been called.  Buffers
the library writes (``out``, states, ``present_state``, ``workspace``) must
already be contiguous with the exact dtype and shape, or the call raises:
a strided or converted copy would receive the results instead of the caller's
tensor.  Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback.  If the shared library is missing
or cannot be loaded, every call raises.

Functions carry the C names:

* :func:`la_initial_state` -- zero streaming state (Keras proposal, "Streaming
  State", get_initial_state).
* :func:`la_forward` -- causal / non-causal attention with masks and streaming
  state (Keras proposal, "Mathematical definition", "Masking").
* :func:`la_forward_noalloc` -- :func:`la_forward` without a workspace, for
  callers that cannot allocate (the library's own per-GPU scratch array).
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
    "LinAttnError", "la_initial_state", "la_forward", "la_forward_noalloc", "la_step", "la_gated_forward",
    "la_gated_step", "la_delta_forward", "la_backward", "la_workspace_size", "la_gated_workspace_size", "library_path", "load_library",
    "EXPORTED_SYMBOLS",
]

EXPORTED_SYMBOLS = (
    "la_initial_state", "la_workspace_size", "la_forward", "la_forward_noalloc", "la_step",
    "la_gated_workspace_size",
    "la_gated_forward", "la_gated_step", "la_delta_forward", "la_delta_workspace_size", "la_backward_workspace_size",
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
        lib.la_forward_noalloc.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, f32, p,
                                           i64, i64, i64, i64, i64, i32, p]
        lib.la_step.argtypes = [p, p, p, p, p, p, p, p, i32, i32, f32, p, i64, i64, i64, i64, i32, p]
        lib.la_gated_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32,
                                                ctypes.POINTER(sz)]
        lib.la_gated_forward.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                         f32, p, sz, p]
        lib.la_gated_step.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i32, f32, p]
        lib.la_delta_forward.argtypes = [p, p, p, p, i32, p, i32, p, p, p, i64, i64, i64, i64, i64, i64,
                                         i32, f32, p, sz, p]
        lib.la_delta_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        lib.la_backward_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        lib.la_backward.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, f32, p, p, p, p, p, i64, i64, i64,
                                    i64, i64, i32, p, sz, p]
        for name in ("la_initial_state", "la_workspace_size", "la_forward", "la_forward_noalloc", "la_step",
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
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("liblinattn works on GPU tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device (%s and %s)" % (dev, t.device))


def _input(t, name, device, dtype=None, shape=None):
    """A read-only argument: checked, then made contiguous.  The caller keeps
    the returned tensor in a local until the library call has been made, so a
    contiguous copy is not handed back to the allocator before the kernels
    that read it are enqueued."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != torch.device(device):
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.contiguous()


def _output(t, name, device, dtype, shape):
    """A buffer the library writes: it must already be contiguous, of the exact
    dtype and shape, on the device (no copy could carry the results back)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != torch.device(device):
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (the library writes it in place)" % name)
    return t


def _workspace(ws, need, device):
    """(tensor, bytes) of the workspace: the caller's (contiguous, on the
    device, at least ``need`` bytes) or a fresh one."""
    if ws is None:
        if need == 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != torch.device(device) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (nbytes, need))
    return ws, nbytes


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
    B, H, Dk, Dv = int(batch_size), int(num_heads), int(key_dim), int(value_dim)
    lib = load_library()
    if out is not None:
        kv, k = out
        dev = kv.device
        _need_cuda(kv, k)
        kv = _output(kv, "kv state", dev, torch.float32, (B, H, Dk, Dv))
        k = _output(k, "k state", dev, torch.float32, (B, H, Dk))
        if use_normalizer and k is None:
            raise ValueError("use_normalizer needs the k state buffer")
    else:
        kv = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=device)
        k = (torch.empty((B, H, Dk), dtype=torch.float32, device=device)
             if use_normalizer else None)
    _check(lib.la_initial_state(_ptr(kv), _ptr(k), B, H, Dk, Dv, _stream(kv.device)),
           "la_initial_state")
    return (kv, k) if use_normalizer else (kv, None)


def _state_pair(state, B, H, Dk, Dv, norm, dev, what, output):
    """(kv, k) of a causal state argument, checked (outputs) or made
    contiguous (inputs)."""
    if state is None:
        return None, None
    kv, k = state
    if not norm and k is not None:
        raise ValueError("%s: use_normalizer=False carries only the kv state" % what)
    if norm and (kv is None) != (k is None):
        raise ValueError("%s: a normalized state needs both kv and k" % what)
    conv = _output if output else _input
    return (conv(kv, what + " kv", dev, torch.float32, (B, H, Dk, Dv)),
            conv(k, what + " k", dev, torch.float32, (B, H, Dk)))


def la_forward(q, k, v, mask=None, state=None, causal=True, feature_map="elu_plus_one",
               use_normalizer=True, eps=1e-6, return_state=False, out=None, state_out=None,
               workspace=None):
    """Linear attention over q,k (B,T,H,Dk), v (B,T,H,Dv).

    ``state``: (kv, k) tuple (k None without the normalizer) or None for zeros.
    ``state_out``: optional (kv, k) buffers for the final state (may be ``state``
    itself for in-place streaming).  Returns ``out`` or ``(out, (kv, k))``.
    """
    return _forward(q, k, v, mask, state, causal, feature_map, use_normalizer, eps, return_state, out,
                    state_out, workspace, False)


def la_forward_noalloc(q, k, v, mask=None, state=None, causal=True, feature_map="elu_plus_one",
                       use_normalizer=True, eps=1e-6, return_state=False, out=None, state_out=None):
    """:func:`la_forward` through the C ABI's allocation-free entry point: the
    library uses its own per-GPU scratch array instead of a workspace.  The
    C entry point allocates nothing; this wrapper still allocates the outputs
    it is not given and the copies it makes (a converted mask, contiguous
    inputs)."""
    return _forward(q, k, v, mask, state, causal, feature_map, use_normalizer, eps, return_state, out,
                    state_out, None, True)


def _forward(q, k, v, mask, state, causal, feature_map, use_normalizer, eps, return_state, out,
             state_out, workspace, noalloc):
    _need_cuda(q, k, v)
    dev = q.device
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be (B,T,H,D)")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype and (B,T,H) with matching Dk")
    q, k, v = _input(q, "q", dev), _input(k, "k", dev), _input(v, "v", dev)
    norm = bool(use_normalizer)
    lib = load_library()
    m = _mask_u8(mask, B, T, dev)
    out = (torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev) if out is None
           else _output(out, "out", dev, q.dtype, (B, T, H, Dv)))
    if not causal and (state is not None or state_out is not None):
        raise ValueError("non-causal attention takes and returns no state")
    s_in_kv, s_in_k = _state_pair(state, B, H, Dk, Dv, norm, dev, "state", output=False)
    s_out_kv = s_out_k = None
    if causal and (return_state or state_out is not None):
        if state_out is not None:
            s_out_kv, s_out_k = _state_pair(state_out, B, H, Dk, Dv, norm, dev, "state_out", output=True)
            if s_out_kv is None:
                raise ValueError("state_out needs the kv buffer")
        else:
            s_out_kv = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
            s_out_k = torch.empty((B, H, Dk), dtype=torch.float32, device=dev) if norm else None
    if noalloc:
        _check(lib.la_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_in_kv), _ptr(s_in_k),
                                      _ptr(s_out_kv), _ptr(s_out_k), int(bool(causal)), _FM[feature_map],
                                      int(norm), float(eps), _ptr(out), B, T, H, Dk, Dv,
                                      _dtype_code(q), _stream(dev)), "la_forward_noalloc")
    else:
        ws_bytes = la_workspace_size(B, T, H, Dk, Dv, q.dtype, causal) if q.dtype in _DT else 0
        ws, wsb = _workspace(workspace, ws_bytes, dev)
        _check(lib.la_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_in_kv), _ptr(s_in_k),
                              _ptr(s_out_kv), _ptr(s_out_k), int(bool(causal)), _FM[feature_map],
                              int(norm), float(eps), _ptr(out), B, T, H, Dk, Dv,
                              _dtype_code(q), _ptr(ws), wsb, _stream(dev)), "la_forward")
    if return_state and causal:
        return out, (s_out_kv, s_out_k)
    return out


def la_step(q, k, v, state, mask=None, feature_map="elu_plus_one", use_normalizer=True, eps=1e-6,
            out=None, state_out=None, in_place=True):
    """One T=1 decode step.  q,k: (B,H,Dk) or (B,1,H,Dk); v likewise.

    Updates ``state`` in place by default (``in_place``; the state buffers must
    then be contiguous float32); otherwise writes to ``state_out`` or fresh
    buffers.  Returns ``(out (B,H,Dv), (kv, k))``.
    """
    _need_cuda(q, k, v)
    dev = q.device
    squeeze = q.dim() == 4
    if squeeze:
        if q.shape[1] != 1 or k.shape[1] != 1 or v.shape[1] != 1:
            raise ValueError("la_step takes one token")
        q, k, v = q[:, 0], k[:, 0], v[:, 0]
    if q.dim() != 3 or k.shape != q.shape or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be (B,H,Dk) and v (B,H,Dv)")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    q, k, v = _input(q, "q", dev), _input(k, "k", dev), _input(v, "v", dev)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    norm = bool(use_normalizer)
    lib = load_library()
    if state is None:
        raise ValueError("a decode step needs a state (la_initial_state)")
    if in_place:
        s_kv, s_k = _state_pair(state, B, H, Dk, Dv, norm, dev, "state", output=True)
        o_kv, o_k = s_kv, s_k
    else:
        s_kv, s_k = _state_pair(state, B, H, Dk, Dv, norm, dev, "state", output=False)
        if state_out is not None:
            o_kv, o_k = _state_pair(state_out, B, H, Dk, Dv, norm, dev, "state_out", output=True)
        else:
            o_kv = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
            o_k = torch.empty((B, H, Dk), dtype=torch.float32, device=dev) if norm else None
    m = None
    if mask is not None:
        m = torch.broadcast_to(torch.as_tensor(mask, device=dev).to(torch.bool).reshape(-1),
                               (B,)).to(torch.uint8).contiguous()
    out = (torch.empty((B, H, Dv), dtype=q.dtype, device=dev) if out is None
           else _output(out, "out", dev, q.dtype, (B, H, Dv)))
    _check(lib.la_step(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_kv), _ptr(s_k), _ptr(o_kv),
                       _ptr(o_k), _FM[feature_map], int(norm), float(eps), _ptr(out),
                       B, H, Dk, Dv, _dtype_code(q), _stream(dev)), "la_step")
    return (out[:, None] if squeeze else out), (o_kv, o_k)


def _packed_heads(q, k, v, Hq, Hkv, ndim):
    """(Dk, Dv) of packed (..., heads*dim) q, k, v, checked."""
    Hq, Hkv = int(Hq), int(Hkv)
    if q.dim() != ndim or k.dim() != ndim or v.dim() != ndim:
        raise ValueError("query, key, value must be %d-D packed tensors" % ndim)
    if Hq < 1 or Hkv < 1 or q.shape[-1] % Hq or k.shape[-1] % Hkv or v.shape[-1] % Hkv:
        raise ValueError("head counts do not divide the packed widths")
    if q.shape[:-1] != k.shape[:-1] or q.shape[:-1] != v.shape[:-1]:
        raise ValueError("query, key, value must share their leading dimensions")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("query, key, value must share one dtype")
    Dk = q.shape[-1] // Hq
    if k.shape[-1] // Hkv != Dk:
        raise ValueError("query and key head sizes differ")
    return Dk, v.shape[-1] // Hkv


def la_gated_forward(query, key, value, q_num_heads, kv_num_heads, decay=None, past_state=None,
                     scale=0.0, out=None, present_state=None, workspace=None):
    """Gated / linear recurrence on packed (B,T,H*D) tensors with GQA.

    ``decay``: log-space, (B,T,Hkv) per kv head or (B,T,Hkv*Dk) per key
    dimension, or None ("linear" rule).
    Returns ``(output (B,T,Hq*Dv), present_state (B,Hkv,Dk,Dv) float32)``.
    """
    _need_cuda(query, key, value, decay, past_state, out, present_state)
    dev = query.device
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    Dk, Dv = _packed_heads(query, key, value, Hq, Hkv, 3)
    B, T, _ = query.shape
    q, k, v = _input(query, "query", dev), _input(key, "key", dev), _input(value, "value", dev)
    lib = load_library()
    per_dim = decay is not None and tuple(decay.shape) == (B, T, Hkv * Dk) and Dk > 1
    if decay is not None and not per_dim and tuple(decay.shape) != (B, T, Hkv):
        raise ValueError("decay must be (B,T,Hkv) (per kv head) or (B,T,Hkv*Dk) (per key dim)")
    g = _input(decay, "decay", dev, q.dtype)
    past = _input(past_state, "past_state", dev, torch.float32, (B, Hkv, Dk, Dv))
    out = (torch.empty((B, T, Hq * Dv), dtype=q.dtype, device=dev) if out is None
           else _output(out, "out", dev, q.dtype, (B, T, Hq * Dv)))
    present_state = (torch.empty((B, Hkv, Dk, Dv), dtype=torch.float32, device=dev)
                     if present_state is None
                     else _output(present_state, "present_state", dev, torch.float32, (B, Hkv, Dk, Dv)))
    ws_bytes = (la_gated_workspace_size(B, T, Hq, Hkv, Dk, Dv, q.dtype, per_dim)
                if q.dtype in _DT else 0)
    ws, wsb = _workspace(workspace, ws_bytes, dev)
    _check(lib.la_gated_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(past),
                                _ptr(present_state), _ptr(out), B, T, Hq, Hkv, Dk, Dv,
                                _dtype_code(q), float(scale), _ptr(ws), wsb, _stream(dev)),
           "la_gated_forward")
    return out, present_state


def la_gated_step(query, key, value, q_num_heads, kv_num_heads, decay=None, past_state=None,
                  scale=0.0, out=None, present_state=None, in_place=False):
    """One token of the gated / linear recurrence: query (B,Hq*Dk) or (B,1,Hq*Dk),
    key / value (B,Hkv*D) or (B,1,Hkv*D), decay (B,Hkv) per kv head or
    (B,Hkv*Dk) per key dim (either with an optional token axis of 1), or None.

    ``in_place`` writes the new state over ``past_state``, which must then be a
    contiguous float32 tensor.  Returns ``(output, present_state (B,Hkv,Dk,Dv)
    float32)``, the output shaped like the query.
    """
    _need_cuda(query, key, value, decay, past_state, out, present_state)
    dev = query.device
    squeeze = query.dim() == 3
    q, k, v, g = query, key, value, decay
    if squeeze:
        if q.shape[1] != 1 or k.dim() != 3 or k.shape[1] != 1 or v.dim() != 3 or v.shape[1] != 1:
            raise ValueError("la_gated_step takes one token")
        q, k, v = q[:, 0], k[:, 0], v[:, 0]
        g = None if g is None else g.reshape(g.shape[0], -1)
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    Dk, Dv = _packed_heads(q, k, v, Hq, Hkv, 2)
    B = q.shape[0]
    q, k, v = _input(q, "query", dev), _input(k, "key", dev), _input(v, "value", dev)
    lib = load_library()
    per_dim = g is not None and tuple(g.shape) == (B, Hkv * Dk) and Dk > 1
    if g is not None and not per_dim and tuple(g.shape) != (B, Hkv):
        raise ValueError("decay must be (B,Hkv) (per kv head) or (B,Hkv*Dk) (per key dim)")
    g = _input(g, "decay", dev, q.dtype)
    sshape = (B, Hkv, Dk, Dv)
    if in_place:
        if past_state is None:
            raise ValueError("in_place needs past_state")
        past = _output(past_state, "past_state (in place)", dev, torch.float32, sshape)
        present_state = past
    else:
        past = _input(past_state, "past_state", dev, torch.float32, sshape)
        present_state = (torch.empty(sshape, dtype=torch.float32, device=dev) if present_state is None
                         else _output(present_state, "present_state", dev, torch.float32, sshape))
    oshape = (B, 1, Hq * Dv) if squeeze else (B, Hq * Dv)
    out = (torch.empty(oshape, dtype=q.dtype, device=dev) if out is None
           else _output(out, "out", dev, q.dtype, oshape))
    _check(lib.la_gated_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(past), _ptr(present_state),
                             _ptr(out), B, Hq, Hkv, Dk, Dv, _dtype_code(q), float(scale), _stream(dev)),
           "la_gated_step")
    return out, present_state


def la_delta_forward(query, key, value, q_num_heads, kv_num_heads, beta, decay=None, past_state=None,
                     scale=0.0, out=None, present_state=None):
    """Delta rule (``decay`` None) or gated delta rule on packed (B,T,H*D) tensors
    with GQA.  ``beta``: (B,T,Hkv) or (B,T,1); ``decay``: log-space, (B,T,Hkv)
    or (B,T,Hkv*Dk).  Returns ``(output (B,T,Hq*Dv), present_state (B,Hkv,Dk,Dv)
    float32)``.
    """
    _need_cuda(query, key, value, beta, decay, past_state, out, present_state)
    dev = query.device
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    Dk, Dv = _packed_heads(query, key, value, Hq, Hkv, 3)
    B, T, _ = query.shape
    q, k, v = _input(query, "query", dev), _input(key, "key", dev), _input(value, "value", dev)
    lib = load_library()
    per_dim = decay is not None and tuple(decay.shape) == (B, T, Hkv * Dk) and Dk > 1
    if decay is not None and not per_dim and tuple(decay.shape) != (B, T, Hkv):
        raise ValueError("decay must be (B,T,Hkv) (per kv head) or (B,T,Hkv*Dk) (per key dim)")
    if beta is None or tuple(beta.shape) not in ((B, T, Hkv), (B, T, 1)):
        raise ValueError("beta must be (B,T,Hkv) or (B,T,1)")
    beta_per_head = tuple(beta.shape) == (B, T, Hkv) and Hkv > 1
    g = _input(decay, "decay", dev, q.dtype)
    be = _input(beta, "beta", dev, q.dtype)
    past = _input(past_state, "past_state", dev, torch.float32, (B, Hkv, Dk, Dv))
    out = (torch.empty((B, T, Hq * Dv), dtype=q.dtype, device=dev) if out is None
           else _output(out, "out", dev, q.dtype, (B, T, Hq * Dv)))
    present_state = (torch.empty((B, Hkv, Dk, Dv), dtype=torch.float32, device=dev)
                     if present_state is None
                     else _output(present_state, "present_state", dev, torch.float32, (B, Hkv, Dk, Dv)))
    n = ctypes.c_size_t(0)
    _check(lib.la_delta_workspace_size(B, T, Hq, Hkv, Dk, Dv, _dtype_code(q), int(per_dim), ctypes.byref(n)),
           "la_delta_workspace_size")
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev) if n.value else None
    _check(lib.la_delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(per_dim), _ptr(be),
                                int(beta_per_head), _ptr(past), _ptr(present_state),
                                _ptr(out), B, T, Hq, Hkv, Dk, Dv, _dtype_code(q), float(scale),
                                _ptr(ws), n.value, _stream(dev)), "la_delta_forward")
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
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q, k, v must be (B,T,H,D)")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or tuple(dout.shape) != tuple(v.shape):
        raise ValueError("q, k (B,T,H,Dk), v and dout (B,T,H,Dv) do not match")
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("q, k, v and dout must share one dtype")
    q, k, v, dout = (_input(q, "q", dev), _input(k, "k", dev), _input(v, "v", dev),
                     _input(dout, "dout", dev))
    norm = bool(use_normalizer)
    lib = load_library()
    m = _mask_u8(mask, B, T, dev)
    # every contiguous copy stays bound to a local until the call is made
    s_kv, s_k = _state_pair(state, B, H, Dk, Dv, norm, dev, "state", output=False)
    g_kv, g_k = _state_pair(dstate, B, H, Dk, Dv, norm, dev, "dstate", output=False)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dS0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    dZ0 = torch.empty((B, H, Dk), dtype=torch.float32, device=dev) if norm else None
    n = ctypes.c_size_t(0)
    _check(lib.la_backward_workspace_size(B, T, H, Dk, Dv, _dtype_code(q), int(norm),
                                          ctypes.byref(n)), "la_backward_workspace_size")
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev)
    _check(lib.la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(s_kv), _ptr(s_k),
                           _ptr(dout), _ptr(g_kv), _ptr(g_k), _FM[feature_map],
                           int(norm), float(eps), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dS0),
                           _ptr(dZ0), B, T, H, Dk, Dv, _dtype_code(q), _ptr(ws), n.value, _stream(dev)),
           "la_backward")
    return dq, dk, dv, (dS0, dZ0)
