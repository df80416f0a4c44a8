"""Seeded synthetic inputs for the five benchmark workloads and the tests.

This module only draws random tensors (and masks) of the workloads' shapes,
dtypes and distributions.  It holds none of the attention arithmetic, so the
oracle and the HIP library can both be fed from it without sharing any code.

Recipes (all values drawn in float32 from a torch generator seeded per tensor,
then rounded to nearest even to the storage dtype):

* ``causal_fp32_small``   B=1 H=2 T=256 D=32, fp32: q,k ~ N(0, 0.5^2), v ~ N(0,1).
* ``causal_bf16_d64``     B=8 H=16 T=2048 D=64, bf16: same distributions.
* ``noncausal_relu_d128`` B=4 H=16 T=16384 D=128, bf16: q,k,v ~ N(0,1); right-padding
  mask, valid length of row b uniform on the integers {T/2, ..., T}.
* ``streaming_d128``      B=256 H=32 D=128, bf16: 4096 prefill tokens and 512
  decode tokens, q,k ~ N(0, 0.5^2), v ~ N(0,1).
* ``gated_gqa_d128``      B=2 T=32768 Hq=32 Hkv=8 D=128, bf16: q,v ~ N(0,1); k drawn
  N(0,1) then L2-normalised per (b,t,kv head) in fp32 before rounding; decay
  g = logsigmoid(x), x ~ N(2,1), computed in fp32 then rounded.
* ``gated_perdim_d128``   the ``gated_gqa_d128`` shapes with a per-key-dim decay
  (B,T,Hkv*D), g = logsigmoid(x), x ~ N(2,1) drawn per element.
* ``gated_delta_d128``    the gated delta rule, B=32 T=4096 Hq=32 Hkv=8 D=128, bf16: q, v,
  unit-norm k and the per-head decay as ``gated_gqa_d128``; beta = sigmoid(x),
  x ~ N(0,1), per (b, t, kv head).
* ``backward_bf16_d64``   the gradients of ``causal_bf16_d64`` (same shapes and
  inputs), with an output gradient dy ~ N(0,1).
* ``gated_step_d128``     the same heads and distributions as a serving batch of
  B=256 sequences decoding 64 tokens one at a time; the fp32 past state is
  drawn N(0, 0.3^2).
* ``delta_step_d128``     ``gated_step_d128`` under the gated delta rule, with
  beta = sigmoid(N(0,1)) per kv head.
* ``gated_perdim_f32_d128`` the per-key-dim gated rule with fp32 inputs at head
  size 128 (B=8 T=2048 Hq=32 Hkv=8): the distributions of ``gated_perdim_d128``.
"""
from __future__ import annotations

import zlib

import torch

WORKLOADS = {
    "causal_fp32_small": dict(B=1, H=2, T=256, D=32, dtype=torch.float32, seed=1),
    "causal_bf16_d64": dict(B=8, H=16, T=2048, D=64, dtype=torch.bfloat16, seed=2),
    "noncausal_relu_d128": dict(B=4, H=16, T=16384, D=128, dtype=torch.bfloat16, seed=3),
    "streaming_d128": dict(B=256, H=32, T=4096, T_decode=512, D=128, dtype=torch.bfloat16, seed=4),
    "gated_gqa_d128": dict(B=2, T=32768, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16, seed=5),
    "gated_step_d128": dict(B=256, T=64, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16, seed=6),
    "gated_perdim_d128": dict(B=2, T=32768, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16, seed=7),
    "gated_delta_d128": dict(B=32, T=4096, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16, seed=8),
    "backward_bf16_d64": dict(B=8, H=16, T=2048, D=64, dtype=torch.bfloat16, seed=9),
    "delta_step_d128": dict(B=256, T=64, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16, seed=10),
    "gated_perdim_f32_d128": dict(B=8, T=2048, Hq=32, Hkv=8, D=128, dtype=torch.float32, seed=11),
}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + zlib.crc32(name.encode())) % (2**63 - 1))
    return g


def normal(shape, std, dtype, device, seed, name, chunk_elems=1 << 28):
    """N(0, std^2) drawn in fp32 then rounded to ``dtype``; generated in slices
    along dim 0 so the fp32 temporary stays bounded for very large tensors."""
    out = torch.empty(shape, dtype=dtype, device=device)
    g = _gen(seed, name, device)
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    rows = max(1, chunk_elems // max(per_row, 1))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        tmp = torch.randn((r1 - r0, per_row), generator=g, device=device, dtype=torch.float32)
        flat[r0:r1] = (tmp * std).to(dtype)
    return out


def qkv(B, T, H, D, dtype, device, seed, q_std=0.5, k_std=0.5, v_std=1.0, tag=""):
    q = normal((B, T, H, D), q_std, dtype, device, seed, "q" + tag)
    k = normal((B, T, H, D), k_std, dtype, device, seed, "k" + tag)
    v = normal((B, T, H, D), v_std, dtype, device, seed, "v" + tag)
    return q, k, v


def right_padding_mask(B, T, device, seed, lo=None, hi=None):
    """(B,T) bool: valid iff t < L_b with L_b uniform on {lo..hi} (default T/2..T)."""
    lo = T // 2 if lo is None else lo
    hi = T if hi is None else hi
    g = _gen(seed, "mask", "cpu")
    L = torch.randint(lo, hi + 1, (B,), generator=g)
    m = torch.arange(T)[None, :] < L[:, None]
    return m.to(device), L


def random_mask(B, T, p_valid, device, seed, tag=""):
    g = _gen(seed, "rmask" + tag, "cpu")
    return (torch.rand((B, T), generator=g) < p_valid).to(device)


def l2_normalized(shape, dtype, device, seed, name):
    """N(0,1) rows normalised to unit L2 norm over the last dim (fp32), then rounded."""
    x = normal(shape, 1.0, torch.float32, device, seed, name)
    x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    return x.to(dtype)


def logsigmoid_decay(shape, dtype, device, seed, mean=2.0, std=1.0):
    x = normal(shape, std, torch.float32, device, seed, "g") + mean
    return torch.nn.functional.logsigmoid(x).to(dtype)


def workload(name: str, device="cpu"):
    """All inputs of a named workload as a dict of tensors on ``device``."""
    w = WORKLOADS[name]
    s, dt = w["seed"], w["dtype"]
    if name in ("gated_gqa_d128", "gated_step_d128", "gated_perdim_d128", "gated_delta_d128", "delta_step_d128",
                "gated_perdim_f32_d128"):
        B, T, Hq, Hkv, D = w["B"], w["T"], w["Hq"], w["Hkv"], w["D"]
        q = normal((B, T, Hq * D), 1.0, dt, device, s, "q")
        k = l2_normalized((B, T, Hkv, D), dt, device, s, "k").reshape(B, T, Hkv * D)
        v = normal((B, T, Hkv * D), 1.0, dt, device, s, "v")
        per_dim = name in ("gated_perdim_d128", "gated_perdim_f32_d128")
        g = logsigmoid_decay((B, T, Hkv * D) if per_dim else (B, T, Hkv), dt, device, s)
        out = dict(q=q, k=k, v=v, decay=g, Hq=Hq, Hkv=Hkv, D=D)
        if name in ("gated_step_d128", "delta_step_d128"):
            out["past"] = normal((B, Hkv, D, D), 0.3, torch.float32, device, s, "past")
        if name in ("gated_delta_d128", "delta_step_d128"):
            out["beta"] = torch.sigmoid(normal((B, T, Hkv), 1.0, torch.float32, device, s, "beta")).to(dt)
        return out
    B, T, H, D = w["B"], w["T"], w["H"], w["D"]
    if name == "noncausal_relu_d128":
        q, k, v = qkv(B, T, H, D, dt, device, s, 1.0, 1.0, 1.0)
        mask, L = right_padding_mask(B, T, device, s)
        return dict(q=q, k=k, v=v, mask=mask, lengths=L)
    q, k, v = qkv(B, T, H, D, dt, device, s)
    out = dict(q=q, k=k, v=v)
    if name == "backward_bf16_d64":
        out["dy"] = normal((B, T, H, D), 1.0, dt, device, s, "dy")
    if name == "streaming_d128":
        Td = w["T_decode"]
        out["q_dec"], out["k_dec"], out["v_dec"] = qkv(B, Td, H, D, dt, device, s, tag="_decode")
    return out
