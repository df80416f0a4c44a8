"""fp64 CPU oracle for kernelized linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the HIP path: the arithmetic lives in ``laoracle.c``
(plain per-token recurrences in double precision, compiled with gcc), and this
module only marshals numpy arrays into it.

Functions follow these passages:

* :func:`causal` -- "[Feature] LinearAttention layer for Keras", sections
  "Mathematical definition / Causal", "Masking / Causal", "Streaming State";
  also the running-sum equations of "Causal Linear Attention" (Brenndoerfer).
* :func:`causal_backward` -- gradients of :func:`causal` (same page, "Stability"
  and "Acceptance": gradient parity, float64 numerical-gradient checks).
* :func:`noncausal` -- same Keras page, "Mathematical definition / Non-causal"
  and "Masking / Non-causal".
* :func:`la_op` -- the "LinearAttention" operator page (ai.onnx, since version
  27), sections "Description", "Inputs", "Attributes": update rules linear,
  gated (per-head or per-key-dim decay), delta, gated_delta; GQA.

Pins (all in ``tests/test_oracle_pins.py``): the operator page's worked examples
(``tests/golden/onnx_examples.json``), the seeded causal-vs-non-causal figure of
the Brenndoerfer page, brute-force quadratic forms on tiny inputs, and closed
forms for special inputs.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "laoracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lock = threading.Lock()
_lib = None

FEATURE_MAPS = {"elu_plus_one": 0, "relu": 1}
RULES = {"linear": 0, "gated": 1, "delta": 2, "gated_delta": 3}


def build(force: bool = False) -> str:
    """Compile laoracle.c into liblaoracle.so with gcc (plain -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, p, u8p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
            lib.oracle_causal.argtypes = [i64] * 5 + [p, p, p, u8p, p, p, ctypes.c_int,
                                                      ctypes.c_int, ctypes.c_double, p, p, p]
            lib.oracle_noncausal.argtypes = [i64] * 5 + [p, p, p, u8p, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_double, p, p, p]
            lib.oracle_la_op.argtypes = [i64] * 6 + [p, p, p, p, p, ctypes.c_int, p, ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_double, p, p]
            lib.oracle_causal_backward.argtypes = [i64] * 5 + [p, p, p, u8p, p, p, p, p, p, ctypes.c_int,
                                                               ctypes.c_int, ctypes.c_double, p, p, p, p, p]
            for f in (lib.oracle_causal, lib.oracle_noncausal, lib.oracle_la_op, lib.oracle_causal_backward):
                f.restype = ctypes.c_int
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def _f64(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mask(m, B, T):
    if m is None:
        return None
    m = np.ascontiguousarray(np.broadcast_to(np.asarray(m).astype(bool), (B, T)).astype(np.uint8))
    return m


def causal(q, k, v, mask=None, S0=None, Z0=None, feature_map="elu_plus_one",
           use_normalizer=True, eps=1e-6):
    """Per-token causal recurrence.  q,k: (B,T,H,Dk); v: (B,T,H,Dv).

    Returns (y (B,T,H,Dv), S (B,H,Dk,Dv), Z (B,H,Dk)), all float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    S0, Z0 = _f64(S0), _f64(Z0)
    if S0 is not None:
        assert S0.shape == (B, H, Dk, Dv)
    if Z0 is not None:
        assert Z0.shape == (B, H, Dk)
    m = _mask(mask, B, T)
    y = np.empty((B, T, H, Dv))
    S = np.empty((B, H, Dk, Dv))
    Z = np.empty((B, H, Dk))
    rc = _load().oracle_causal(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(S0),
                               _ptr(Z0), FEATURE_MAPS[feature_map], int(bool(use_normalizer)),
                               float(eps), _ptr(y), _ptr(S), _ptr(Z))
    if rc:
        raise ValueError("oracle_causal rejected its arguments (%d)" % rc)
    return y, S, Z


def causal_backward(q, k, v, dy, mask=None, S0=None, Z0=None, dS_T=None, dZ_T=None,
                    feature_map="elu_plus_one", use_normalizer=True, eps=1e-6):
    """Gradients of :func:`causal` for the loss sum(dy * y) + sum(dS_T * S_T) +
    sum(dZ_T * Z_T), by reverse-mode differentiation of the per-token recurrence
    (Keras proposal, "Stability": float64 numerical-gradient checks; "Acceptance":
    recurrent/parallel gradient parity).

    Returns (dq, dk, dv, dS0, dZ0), float64.
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv) and dy.shape == (B, T, H, Dv)
    S0, Z0, dS_T, dZ_T = _f64(S0), _f64(Z0), _f64(dS_T), _f64(dZ_T)
    m = _mask(mask, B, T)
    dq = np.empty((B, T, H, Dk))
    dk = np.empty((B, T, H, Dk))
    dv = np.empty((B, T, H, Dv))
    dS0 = np.empty((B, H, Dk, Dv))
    dZ0 = np.empty((B, H, Dk))
    rc = _load().oracle_causal_backward(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(S0),
                                        _ptr(Z0), _ptr(dy), _ptr(dS_T), _ptr(dZ_T),
                                        FEATURE_MAPS[feature_map], int(bool(use_normalizer)),
                                        float(eps), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dS0), _ptr(dZ0))
    if rc:
        raise ValueError("oracle_causal_backward rejected its arguments (%d)" % rc)
    return dq, dk, dv, dS0, dZ0


def noncausal(q, k, v, mask=None, feature_map="elu_plus_one", use_normalizer=True, eps=1e-6):
    """Non-causal closed form.  Returns (y, S, Z), float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    m = _mask(mask, B, T)
    y = np.empty((B, T, H, Dv))
    S = np.empty((B, H, Dk, Dv))
    Z = np.empty((B, H, Dk))
    rc = _load().oracle_noncausal(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                                  FEATURE_MAPS[feature_map], int(bool(use_normalizer)),
                                  float(eps), _ptr(y), _ptr(S), _ptr(Z))
    if rc:
        raise ValueError("oracle_noncausal rejected its arguments (%d)" % rc)
    return y, S, Z


def la_op(query, key, value, q_num_heads, kv_num_heads, update_rule="linear",
          past_state=None, decay=None, beta=None, scale=0.0):
    """Operator form on packed (B,T,heads*dim) tensors.

    Returns (output (B,T,Hq*Dv), present_state (B,Hkv,Dk,Dv)), float64.
    ``scale == 0`` means 1/sqrt(Dk) with Dk = query.shape[-1] / q_num_heads.
    """
    q, k, v = _f64(query), _f64(key), _f64(value)
    B, T, qw = q.shape
    Hq, Hkv = int(q_num_heads), int(kv_num_heads)
    if Hq < 1 or Hkv < 1 or Hq % Hkv or qw % Hq or k.shape[-1] % Hkv or v.shape[-1] % Hkv:
        raise ValueError("bad head counts")
    Dk = qw // Hq
    Dv = v.shape[-1] // Hkv
    assert k.shape == (B, T, Hkv * Dk) and v.shape == (B, T, Hkv * Dv)
    if scale == 0.0:
        scale = 1.0 / np.sqrt(Dk)
    decay_per_dim = 0
    if decay is not None:
        decay = _f64(decay)
        if decay.shape == (B, T, Hkv * Dk) and Dk != 1:
            decay_per_dim = 1
        elif decay.shape != (B, T, Hkv):
            raise ValueError("decay must be (B,T,Hkv) or (B,T,Hkv*Dk)")
    beta_per_head = 1
    if beta is not None:
        beta = _f64(beta)
        if beta.shape == (B, T, 1) and Hkv != 1:
            beta_per_head = 0
        elif beta.shape == (B, T, 1):
            beta_per_head = 0
        elif beta.shape != (B, T, Hkv):
            raise ValueError("beta must be (B,T,Hkv) or (B,T,1)")
    past = _f64(past_state)
    if past is not None:
        assert past.shape == (B, Hkv, Dk, Dv)
    out = np.empty((B, T, Hq * Dv))
    present = np.empty((B, Hkv, Dk, Dv))
    rc = _load().oracle_la_op(B, T, Hq, Hkv, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(past),
                              _ptr(decay), decay_per_dim, _ptr(beta), beta_per_head,
                              RULES[update_rule], float(scale), _ptr(out), _ptr(present))
    if rc:
        raise ValueError("oracle_la_op rejected its arguments (%d)" % rc)
    return out, present
