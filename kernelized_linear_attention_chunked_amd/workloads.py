"""Drivers for the benchmark workloads.

Each driver allocates the seeded inputs (from ``synth``), the outputs, state
and workspace on the device once, precomputes the raw pointers, and issues the
call sequence of one step through the C ABI on torch's current stream.  No
arithmetic of the method lives here.
"""
from __future__ import annotations

import ctypes

import torch

import synth

from . import _check, _stream, la_gated_workspace_size, la_workspace_size, load_library

P = ctypes.c_void_p


def _p(t):
    return None if t is None else P(t.data_ptr())


class StreamingD128:
    """Streaming causal elu+1 normalized attention, B=256 H=32 Dk=Dv=128, bf16:
    4096 prefill tokens as four 1024-token calls chained through an fp32
    state updated in place, then 512 T=1 decode steps on the same state."""

    name = "streaming_d128"

    def __init__(self, device="cuda:0", chunk=1024, keep_full=False, eps=1e-6):
        w = synth.WORKLOADS[self.name]
        self.B, self.H, self.T, self.Td, self.D = w["B"], w["H"], w["T"], w["T_decode"], w["D"]
        self.chunk, self.eps, self.device = chunk, eps, device
        B, H, T, Td, D = self.B, self.H, self.T, self.Td, self.D
        inp = synth.workload(self.name, device)
        n = T // chunk
        self.qc = [inp["q"][:, i * chunk:(i + 1) * chunk].contiguous() for i in range(n)]
        self.kc = [inp["k"][:, i * chunk:(i + 1) * chunk].contiguous() for i in range(n)]
        self.vc = [inp["v"][:, i * chunk:(i + 1) * chunk].contiguous() for i in range(n)]
        # decode inputs stored step-major so that every step reads a contiguous slab
        self.qd = inp["q_dec"].transpose(0, 1).contiguous()
        self.kd = inp["k_dec"].transpose(0, 1).contiguous()
        self.vd = inp["v_dec"].transpose(0, 1).contiguous()
        self.full = (inp["q"], inp["k"], inp["v"]) if keep_full else None
        del inp
        self.kv = torch.empty((B, H, D, D), dtype=torch.float32, device=device)
        self.z = torch.empty((B, H, D), dtype=torch.float32, device=device)
        self.out_c = [torch.empty((B, chunk, H, D), dtype=torch.bfloat16, device=device)
                      for _ in range(n)]
        self.out_d = torch.empty((Td, B, H, D), dtype=torch.bfloat16, device=device)
        assert la_workspace_size(B, chunk, H, D, D, torch.bfloat16, True) == 0
        self.lib = load_library()
        st = self.qd[0].numel() * 2
        self._dq = [P(self.qd.data_ptr() + t * st) for t in range(Td)]
        self._dk = [P(self.kd.data_ptr() + t * st) for t in range(Td)]
        self._dv = [P(self.vd.data_ptr() + t * st) for t in range(Td)]
        self._do = [P(self.out_d.data_ptr() + t * st) for t in range(Td)]

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def reset_state(self):
        _check(self.lib.la_initial_state(_p(self.kv), _p(self.z), self.B, self.H, self.D, self.D,
                                         _stream(self.device)), "la_initial_state")

    def prefill_call(self, i, stream=None):
        s = stream or _stream(self.device)
        kv, z = _p(self.kv), _p(self.z)
        _check(self.lib.la_forward(_p(self.qc[i]), _p(self.kc[i]), _p(self.vc[i]), None, kv, z, kv,
                                   z, 1, 0, 1, self.eps, _p(self.out_c[i]), self.B, self.chunk,
                                   self.H, self.D, self.D, 1, None, 0, s), "la_forward")

    def decode_call(self, t, stream=None):
        s = stream or _stream(self.device)
        kv, z = _p(self.kv), _p(self.z)
        _check(self.lib.la_step(self._dq[t], self._dk[t], self._dv[t], None, kv, z, kv, z, 0, 1,
                                self.eps, self._do[t], self.B, self.H, self.D, self.D, 1, s),
               "la_step")

    def prefill(self):
        self.reset_state()
        for i in range(len(self.qc)):
            self.prefill_call(i)

    def decode(self):
        for t in range(self.Td):
            self.decode_call(t)

    def step(self):
        self.prefill()
        self.decode()


class CausalBf16D64:
    """Causal elu+1 normalized full-sequence prefill, B=8 H=16 T=2048 D=64, bf16,
    returning the fp32 state."""

    name = "causal_bf16_d64"

    def __init__(self, device="cuda:0", eps=1e-6):
        w = synth.WORKLOADS[self.name]
        self.B, self.H, self.T, self.D = w["B"], w["H"], w["T"], w["D"]
        self.device, self.eps = device, eps
        inp = synth.workload(self.name, device)
        self.q, self.k, self.v = inp["q"], inp["k"], inp["v"]
        B, H, T, D = self.B, self.H, self.T, self.D
        self.out = torch.empty_like(self.q)
        self.kv = torch.empty((B, H, D, D), dtype=torch.float32, device=device)
        self.z = torch.empty((B, H, D), dtype=torch.float32, device=device)
        n = la_workspace_size(B, T, H, D, D, torch.bfloat16, True)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = n
        self.lib = load_library()

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def step(self):
        _check(self.lib.la_forward(_p(self.q), _p(self.k), _p(self.v), None, None, None,
                                   _p(self.kv), _p(self.z), 1, 0, 1, self.eps, _p(self.out), self.B,
                                   self.T, self.H, self.D, self.D, 1, _p(self.ws), self.ws_bytes,
                                   _stream(self.device)), "la_forward")


class NonCausalReluD128:
    """Non-causal relu+eps normalized attention with a right-padding mask,
    B=4 H=16 T=16384 D=128, bf16."""

    name = "noncausal_relu_d128"

    def __init__(self, device="cuda:0", eps=1e-6):
        w = synth.WORKLOADS[self.name]
        self.B, self.H, self.T, self.D = w["B"], w["H"], w["T"], w["D"]
        self.device, self.eps = device, eps
        inp = synth.workload(self.name, device)
        self.q, self.k, self.v = inp["q"], inp["k"], inp["v"]
        self.mask = inp["mask"].to(torch.uint8).contiguous()
        self.lengths = inp["lengths"]
        B, H, T, D = self.B, self.H, self.T, self.D
        self.out = torch.empty_like(self.q)
        n = la_workspace_size(B, T, H, D, D, torch.bfloat16, False)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = n
        self.lib = load_library()

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def step(self):
        _check(self.lib.la_forward(_p(self.q), _p(self.k), _p(self.v), _p(self.mask), None, None,
                                   None, None, 0, 1, 1, self.eps, _p(self.out), self.B, self.T,
                                   self.H, self.D, self.D, 1, _p(self.ws), self.ws_bytes,
                                   _stream(self.device)), "la_forward")


class GatedGqaD128:
    """Gated recurrence with per-head scalar decay and GQA, B=2 T=32768 Hq=32
    Hkv=8 D=128, bf16, scale 1/sqrt(128), zero past state."""

    name = "gated_gqa_d128"
    per_dim = 0
    io = 1  # la_dtype of the inputs

    def __init__(self, device="cuda:0"):
        w = synth.WORKLOADS[self.name]
        self.B, self.T, self.Hq, self.Hkv, self.D = w["B"], w["T"], w["Hq"], w["Hkv"], w["D"]
        self.device = device
        inp = synth.workload(self.name, device)
        self.q, self.k, self.v, self.g = inp["q"], inp["k"], inp["v"], inp["decay"]
        B, T, D = self.B, self.T, self.D
        self.out = torch.empty_like(self.q)
        self.present = torch.empty((B, self.Hkv, D, D), dtype=torch.float32, device=device)
        n = la_gated_workspace_size(B, T, self.Hq, self.Hkv, D, D, self.q.dtype, bool(self.per_dim))
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = n
        self.scale = 1.0 / (D ** 0.5)
        self.lib = load_library()

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def step(self):
        _check(self.lib.la_gated_forward(_p(self.q), _p(self.k), _p(self.v), _p(self.g), self.per_dim, None,
                                         _p(self.present), _p(self.out), self.B, self.T, self.Hq,
                                         self.Hkv, self.D, self.D, self.io, self.scale, _p(self.ws),
                                         self.ws_bytes, _stream(self.device)), "la_gated_forward")


class GatedPerdimD128(GatedGqaD128):
    """The same recurrence with a per-key-dim decay (B,T,Hkv*D)."""

    name = "gated_perdim_d128"
    per_dim = 1


class GatedPerdimF32D128(GatedGqaD128):
    """The per-key-dim gated rule with fp32 inputs at head size 128, B=8 T=2048
    Hq=32 Hkv=8: the whole-sequence token-by-token path (one launch)."""

    name = "gated_perdim_f32_d128"
    per_dim = 1
    io = 0


class GatedDeltaD128:
    """Gated delta rule with per-head decay and beta, GQA, B=32 T=4096 Hq=32
    Hkv=8 D=128, bf16, scale 1/sqrt(128), zero past state."""

    name = "gated_delta_d128"

    def __init__(self, device="cuda:0"):
        w = synth.WORKLOADS[self.name]
        self.B, self.T, self.Hq, self.Hkv, self.D = w["B"], w["T"], w["Hq"], w["Hkv"], w["D"]
        self.device = device
        inp = synth.workload(self.name, device)
        self.q, self.k, self.v, self.g, self.beta = inp["q"], inp["k"], inp["v"], inp["decay"], inp["beta"]
        B, T, D = self.B, self.T, self.D
        self.out = torch.empty_like(self.q)
        self.present = torch.empty((B, self.Hkv, D, D), dtype=torch.float32, device=device)
        self.scale = 1.0 / (D ** 0.5)
        self.lib = load_library()

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def step(self):
        _check(self.lib.la_delta_forward(_p(self.q), _p(self.k), _p(self.v), _p(self.g), 0, _p(self.beta),
                                         1, None, _p(self.present), _p(self.out), self.B, self.T, self.Hq,
                                         self.Hkv, self.D, self.D, 1, self.scale, None, 0, _stream(self.device)),
               "la_delta_forward")


class BackwardBf16D64:
    """Gradients of the causal elu+1 normalized attention, B=8 H=16 T=2048 D=64,
    bf16 (dq, dk, dv and the initial-state gradient)."""

    name = "backward_bf16_d64"

    def __init__(self, device="cuda:0", eps=1e-6):
        w = synth.WORKLOADS[self.name]
        self.B, self.H, self.T, self.D = w["B"], w["H"], w["T"], w["D"]
        self.device, self.eps = device, eps
        inp = synth.workload(self.name, device)
        self.q, self.k, self.v, self.dy = inp["q"], inp["k"], inp["v"], inp["dy"]
        B, H, T, D = self.B, self.H, self.T, self.D
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.dS0 = torch.empty((B, H, D, D), dtype=torch.float32, device=device)
        self.dZ0 = torch.empty((B, H, D), dtype=torch.float32, device=device)
        self.lib = load_library()
        n = ctypes.c_size_t(0)
        _check(self.lib.la_backward_workspace_size(B, T, H, D, D, 1, 1, ctypes.byref(n)),
               "la_backward_workspace_size")
        self.ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=device)
        self.ws_bytes = n.value

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def step(self):
        _check(self.lib.la_backward(_p(self.q), _p(self.k), _p(self.v), None, None, None, _p(self.dy), None, None,
                                    0, 1, self.eps, _p(self.dq), _p(self.dk), _p(self.dv), _p(self.dS0),
                                    _p(self.dZ0), self.B, self.T, self.H, self.D, self.D, 1, _p(self.ws),
                                    self.ws_bytes, _stream(self.device)), "la_backward")


class GatedStepD128:
    """Gated GQA decode: B=256 sequences, Hq=32 Hkv=8 D=128, bf16, 64 one-token
    steps per step() updating the fp32 state in place."""

    name = "gated_step_d128"

    def __init__(self, device="cuda:0"):
        w = synth.WORKLOADS[self.name]
        self.B, self.T, self.Hq, self.Hkv, self.D = w["B"], w["T"], w["Hq"], w["Hkv"], w["D"]
        self.device = device
        inp = synth.workload(self.name, device)
        B, T, D = self.B, self.T, self.D
        # step-major copies: token t of every sequence is one contiguous block
        self.q = inp["q"].transpose(0, 1).contiguous()
        self.k = inp["k"].transpose(0, 1).contiguous()
        self.v = inp["v"].transpose(0, 1).contiguous()
        self.g = inp["decay"].transpose(0, 1).contiguous()
        self.state = inp["past"]
        self.out = torch.empty((T, B, self.Hq * D), dtype=torch.bfloat16, device=device)
        self.scale = 1.0 / (D ** 0.5)
        self.lib = load_library()

    @property
    def prefill_tokens(self):
        return self.B * self.T

    def decode_call(self, t, stream=None):
        _check(self.lib.la_gated_step(_p(self.q[t]), _p(self.k[t]), _p(self.v[t]), _p(self.g[t]), 0,
                                      _p(self.state), _p(self.state), _p(self.out[t]), self.B,
                                      self.Hq, self.Hkv, self.D, self.D, 1, self.scale,
                                      _stream(self.device) if stream is None else stream),
               "la_gated_step")

    def step(self):
        for t in range(self.T):
            self.decode_call(t)


class DeltaStepD128(GatedStepD128):
    """Gated delta decode: the shapes of gated_step_d128, beta per kv head, 64
    one-token steps per step() updating the fp32 state in place."""

    name = "delta_step_d128"

    def __init__(self, device="cuda:0"):
        super().__init__(device)
        inp = synth.workload(self.name, device)
        self.beta = inp["beta"].transpose(0, 1).contiguous()

    def decode_call(self, t, stream=None):
        _check(self.lib.la_delta_forward(_p(self.q[t]), _p(self.k[t]), _p(self.v[t]), _p(self.g[t]), 0,
                                         _p(self.beta[t]), 1, _p(self.state), _p(self.state),
                                         _p(self.out[t]), self.B, 1, self.Hq, self.Hkv, self.D, self.D,
                                         1, self.scale, None, 0, _stream(self.device) if stream is None else stream),
               "la_delta_forward")


DRIVERS = {c.name: c for c in (StreamingD128, CausalBf16D64, NonCausalReluD128, GatedGqaD128,
                               GatedPerdimD128, GatedPerdimF32D128, GatedDeltaD128, BackwardBf16D64,
                               GatedStepD128, DeltaStepD128)}
