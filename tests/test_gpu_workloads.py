"""Parity at the five benchmark workloads' full sizes, in the call sequences the
bench times (kernelized_linear_attention_chunked_amd.workloads).  Where the
fp64 oracle cannot cover the whole workload in seconds, seeded samples of
(batch, head) units are checked element by element over their full length, and
properties that hold at any size (masked rows exactly zero, chunked == full)
are checked on every element.

Tolerance: floored relative error (tests/_util.py) <= 1e-4 for fp32 inputs,
<= 2e-2 for bf16 inputs with fp32 state."""
import numpy as np
import pytest
import torch

import oracle
import synth
import kernelized_linear_attention_chunked_amd as la
from kernelized_linear_attention_chunked_amd import workloads
from _util import assert_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _units(B, H, n, seed):
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (B - 1, H - 1)}
    while len(picks) < n:
        picks.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(picks)


def _gpu_compare(x, y, rows=16):
    """(max abs difference, floored relative error) of x against y, on the GPU,
    a few batch rows at a time to bound the temporaries."""
    rms = torch.sqrt(sum((y[i:i + rows].float() ** 2).sum() for i in range(0, y.shape[0], rows))
                     / y.numel())
    gap, err = 0.0, 0.0
    for i in range(0, y.shape[0], rows):
        d = (x[i:i + rows].float() - y[i:i + rows].float()).abs()
        gap = max(gap, d.max().item())
        err = max(err, (d / torch.maximum(y[i:i + rows].float().abs(), rms)).max().item())
    return gap, err


def test_causal_fp32_small_full():
    inp = synth.workload("causal_fp32_small", DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    print("workload causal_fp32_small", tuple(q.shape), flush=True)
    y, (S, Z) = la.la_forward(q, k, v, causal=True, return_state=True)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    for x, r, n in ((y, yo, "out"), (S, So, "S"), (Z, Zo, "Z")):
        print(n, "err %.3e" % assert_close(x, r, 1e-4, n))


def test_causal_bf16_d64_full():
    d = workloads.CausalBf16D64(DEV)
    print("workload causal_bf16_d64", tuple(d.q.shape), "workspace", d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(d.q), f64(d.k), f64(d.v))
    for x, r, n in ((d.out, yo, "out"), (d.kv, So, "S"), (d.z, Zo, "Z")):
        print(n, "err %.3e" % assert_close(x, r, 2e-2, n))


def test_noncausal_relu_d128_full():
    d = workloads.NonCausalReluD128(DEV)
    print("workload noncausal_relu_d128", tuple(d.q.shape), "lengths", d.lengths.tolist(), flush=True)
    d.step()
    torch.cuda.synchronize()
    valid = d.mask.bool()
    # every masked query row is exactly zero, everywhere
    assert torch.count_nonzero(d.out[~valid]) == 0
    assert torch.isfinite(d.out.float()).all()
    for b, h in _units(d.B, d.H, 6, 3):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        yo, _, _ = oracle.noncausal(f64(d.q[sl]), f64(d.k[sl]), f64(d.v[sl]),
                                    d.mask[b:b + 1].cpu().numpy(), "relu", True, 1e-6)
        e = assert_close(d.out[sl], yo, 2e-2, "out unit %d,%d" % (b, h))
        print("unit", (b, h), "err %.3e" % e)


def test_streaming_d128_full():
    d = workloads.StreamingD128(DEV, keep_full=True)
    print("workload streaming_d128: 4 x", tuple(d.qc[0].shape), "+", d.Td, "decode steps", flush=True)
    d.step()
    y_chunked = torch.cat(d.out_c, 1)
    S_stream, Z_stream = d.kv.clone(), d.z.clone()
    # one full 4096-token pass must equal the four chained 1024-token calls
    q, k, v = d.full
    y_full, (S_full, Z_full) = la.la_forward(q, k, v, causal=True, return_state=True)
    torch.cuda.synchronize()
    gap, e_cf = _gpu_compare(y_chunked, y_full)
    print("chunked vs full: max abs %.3e, floored rel %.3e" % (gap, e_cf))
    assert e_cf <= 2e-2
    # sampled units against the oracle over all 4096 + 512 tokens
    for b, h in _units(d.B, d.H, 6, 4):
        qa = torch.cat([q[b, :, h], d.qd[:, b, h]], 0)[None, :, None]
        ka = torch.cat([k[b, :, h], d.kd[:, b, h]], 0)[None, :, None]
        va = torch.cat([v[b, :, h], d.vd[:, b, h]], 0)[None, :, None]
        yo, So, Zo = oracle.causal(f64(qa), f64(ka), f64(va))
        T = d.T
        e1 = assert_close(y_chunked[b, :, h], yo[0, :T, 0], 2e-2, "prefill %d,%d" % (b, h))
        e2 = assert_close(y_full[b, :, h], yo[0, :T, 0], 2e-2, "full pass %d,%d" % (b, h))
        e3 = assert_close(d.out_d[:, b, h], yo[0, T:, 0], 2e-2, "decode %d,%d" % (b, h))
        e4 = assert_close(S_stream[b, h], So[0, 0], 2e-2, "S %d,%d" % (b, h))
        e5 = assert_close(Z_stream[b, h], Zo[0, 0], 2e-2, "Z %d,%d" % (b, h))
        print("unit", (b, h), "prefill %.2e full %.2e decode %.2e S %.2e Z %.2e"
              % (e1, e2, e3, e4, e5))
        # the state after the full pass matches the oracle's state after 4096 tokens
        _, So4, Zo4 = oracle.causal(f64(qa[:, :T]), f64(ka[:, :T]), f64(va[:, :T]))
        assert_close(S_full[b, h], So4[0, 0], 2e-2, "S full")
        assert_close(Z_full[b, h], Zo4[0, 0], 2e-2, "Z full")


def test_gated_gqa_d128_full():
    d = workloads.GatedGqaD128(DEV)
    G = d.Hq // d.Hkv
    print("workload gated_gqa_d128", tuple(d.q.shape), "workspace", d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    D = d.D
    for b, j in _units(d.B, d.Hkv, 3, 5):
        qs = d.q[b:b + 1, :, j * G * D:(j + 1) * G * D]
        ks = d.k[b:b + 1, :, j * D:(j + 1) * D]
        vs = d.v[b:b + 1, :, j * D:(j + 1) * D]
        gs = d.g[b:b + 1, :, j:j + 1]
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated", decay=f64(gs),
                              scale=d.scale)
        e1 = assert_close(d.out[b:b + 1, :, j * G * D:(j + 1) * G * D], oo, 2e-2, "out %d,%d" % (b, j))
        e2 = assert_close(d.present[b:b + 1, j:j + 1], po, 2e-2, "present %d,%d" % (b, j))
        print("unit", (b, j), "out %.2e present %.2e" % (e1, e2))


def test_gated_step_d128_full():
    """The gated decode workload: 64 one-token steps of B=256 sequences, in place.
    Sampled (batch, kv head) units are checked against one oracle run over the
    64 tokens from the same past state."""
    d = workloads.GatedStepD128(DEV)
    G, D = d.Hq // d.Hkv, d.D
    past = d.state.clone()
    print("workload gated_step_d128", (d.B, d.T, d.Hq * D), "state", tuple(d.state.shape), flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all() and torch.isfinite(d.state).all()
    for b, j in _units(d.B, d.Hkv, 6, 6):
        qs = d.q[:, b:b + 1, j * G * D:(j + 1) * G * D].transpose(0, 1)
        ks = d.k[:, b:b + 1, j * D:(j + 1) * D].transpose(0, 1)
        vs = d.v[:, b:b + 1, j * D:(j + 1) * D].transpose(0, 1)
        gs = d.g[:, b:b + 1, j:j + 1].transpose(0, 1)
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated", decay=f64(gs),
                              past_state=f64(past[b:b + 1, j:j + 1]), scale=d.scale)
        out = d.out[:, b:b + 1, j * G * D:(j + 1) * G * D].transpose(0, 1)
        e1 = assert_close(out, oo, 2e-2, "out %d,%d" % (b, j))
        e2 = assert_close(d.state[b:b + 1, j:j + 1], po, 2e-2, "state %d,%d" % (b, j))
        print("unit", (b, j), "out %.2e state %.2e" % (e1, e2))


def test_delta_step_d128_full():
    """The gated delta decode workload: 64 one-token steps of B=256 sequences,
    in place, beta per kv head.  Sampled (batch, kv head) units are checked
    against one oracle run over the 64 tokens from the same past state."""
    d = workloads.DeltaStepD128(DEV)
    G, D = d.Hq // d.Hkv, d.D
    past = d.state.clone()
    print("workload delta_step_d128", (d.B, d.T, d.Hq * D), "state", tuple(d.state.shape), flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all() and torch.isfinite(d.state).all()
    for b, j in _units(d.B, d.Hkv, 6, 6):
        qs = d.q[:, b:b + 1, j * G * D:(j + 1) * G * D].transpose(0, 1)
        ks = d.k[:, b:b + 1, j * D:(j + 1) * D].transpose(0, 1)
        vs = d.v[:, b:b + 1, j * D:(j + 1) * D].transpose(0, 1)
        gs = d.g[:, b:b + 1, j:j + 1].transpose(0, 1)
        bs = d.beta[:, b:b + 1, j:j + 1].transpose(0, 1)
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated_delta", decay=f64(gs), beta=f64(bs),
                              past_state=f64(past[b:b + 1, j:j + 1]), scale=d.scale)
        out = d.out[:, b:b + 1, j * G * D:(j + 1) * G * D].transpose(0, 1)
        e1 = assert_close(out, oo, 2e-2, "out %d,%d" % (b, j))
        e2 = assert_close(d.state[b:b + 1, j:j + 1], po, 2e-2, "state %d,%d" % (b, j))
        print("unit", (b, j), "out %.2e state %.2e" % (e1, e2))

def test_gated_perdim_d128_full():
    """The per-key-dim decay at the GQA workload's sizes (split sequences):
    sampled (batch, kv head) units against the oracle over all 32768 tokens."""
    d = workloads.GatedPerdimD128(DEV)
    G, D = d.Hq // d.Hkv, d.D
    print("workload gated_perdim_d128", tuple(d.q.shape), "decay", tuple(d.g.shape), "workspace",
          d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    for b, j in _units(d.B, d.Hkv, 3, 7):
        qs = d.q[b:b + 1, :, j * G * D:(j + 1) * G * D]
        ks = d.k[b:b + 1, :, j * D:(j + 1) * D]
        vs = d.v[b:b + 1, :, j * D:(j + 1) * D]
        gs = d.g[b:b + 1, :, j * D:(j + 1) * D]
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated", decay=f64(gs), scale=d.scale)
        e1 = assert_close(d.out[b:b + 1, :, j * G * D:(j + 1) * G * D], oo, 2e-2, "out %d,%d" % (b, j))
        e2 = assert_close(d.present[b:b + 1, j:j + 1], po, 2e-2, "present %d,%d" % (b, j))
        print("unit", (b, j), "out %.2e present %.2e" % (e1, e2))


def test_gated_delta_d128_full():
    """The gated delta rule at B=32 T=4096 Hq=32 Hkv=8 D=128: sampled (batch, kv
    head) units against the oracle over all 4096 tokens."""
    d = workloads.GatedDeltaD128(DEV)
    G, D = d.Hq // d.Hkv, d.D
    print("workload gated_delta_d128", tuple(d.q.shape), flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    for b, j in _units(d.B, d.Hkv, 3, 8):
        qs = d.q[b:b + 1, :, j * G * D:(j + 1) * G * D]
        ks = d.k[b:b + 1, :, j * D:(j + 1) * D]
        vs = d.v[b:b + 1, :, j * D:(j + 1) * D]
        gs = d.g[b:b + 1, :, j:j + 1]
        bs = d.beta[b:b + 1, :, j:j + 1]
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated_delta", decay=f64(gs), beta=f64(bs),
                              scale=d.scale)
        e1 = assert_close(d.out[b:b + 1, :, j * G * D:(j + 1) * G * D], oo, 2e-2, "out %d,%d" % (b, j))
        e2 = assert_close(d.present[b:b + 1, j:j + 1], po, 2e-2, "present %d,%d" % (b, j))
        print("unit", (b, j), "out %.2e present %.2e" % (e1, e2))


def test_backward_bf16_d64_full():
    """The backward workload (B=8 H=16 T=2048 D=64 bf16): sampled (batch, head)
    units against the oracle backward over all 2048 tokens."""
    d = workloads.BackwardBf16D64(DEV)
    print("workload backward_bf16_d64", tuple(d.q.shape), "workspace", d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    for t in (d.dq, d.dk, d.dv):
        assert torch.isfinite(t.float()).all()
    for b, h in _units(d.B, d.H, 3, 9):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(d.q[sl]), f64(d.k[sl]), f64(d.v[sl]), f64(d.dy[sl]))
        errs = [assert_close(x, y, 2e-2, "%s %d,%d" % (w, b, h))
                for x, y, w in ((d.dq[sl], oq, "dq"), (d.dk[sl], ok_, "dk"), (d.dv[sl], ov, "dv"),
                                (d.dS0[b:b + 1, h:h + 1], oS, "dS0"), (d.dZ0[b:b + 1, h:h + 1], oZ, "dZ0"))]
        print("unit", (b, h), " ".join("%.2e" % e for e in errs))
