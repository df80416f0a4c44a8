"""Parity at the benchmark workloads' full sizes, in the call sequences the
bench times (kernelized_linear_attention_chunked_amd.workloads), against the
fp64 oracle.

Coverage: every (batch, head) unit of every workload is compared element by
element, except the streaming workload (B=256 H=32 over 4096 + 512 tokens,
8192 units), where 16 whole batch rows (512 units, rows 0 and 255 among them)
are compared over all 4608 tokens: the chained 4 x 1024 prefill, the single
4096-token pass, all 512 decode outputs and the states after 4096 and 4608
tokens.  The remaining units are covered by properties that hold at any size:
the chunked stream equals the full pass, every output is finite.

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


def _rows(B, n, seed):
    """n distinct batch rows, the first and the last among them."""
    rng = np.random.default_rng(seed)
    picks = {0, B - 1}
    while len(picks) < min(n, B):
        picks.add(int(rng.integers(B)))
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


def _per_unit_check(x, y, tol, what, unit_axes):
    """Floored relative error of every unit on its own (the RMS floor taken per
    unit, so a unit with small outputs is not hidden by the others), plus the
    whole-tensor figure.  ``unit_axes``: the axes that index a unit."""
    x, y = f64(x), f64(y)
    e_all = assert_close(x, y, tol, what)
    red = tuple(i for i in range(y.ndim) if i not in unit_axes)
    rms = np.sqrt(np.mean(y * y, axis=red, keepdims=True))
    rms = np.where(rms == 0.0, 1.0, rms)
    e_unit = np.max(np.abs(x - y) / np.maximum(np.abs(y), rms), axis=red)
    worst = float(e_unit.max())
    assert worst <= tol, "%s: worst unit %s error %.3e" % (
        what, np.unravel_index(int(np.argmax(e_unit)), e_unit.shape), worst)
    return e_all, worst


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
    for x, r, n, ax in ((d.out, yo, "out", (0, 2)), (d.kv, So, "S", (0, 1)), (d.z, Zo, "Z", (0, 1))):
        print(n, "err %.3e worst unit %.3e" % _per_unit_check(x, r, 2e-2, n, ax))


def test_noncausal_relu_d128_full():
    """All 64 (batch, head) units over all 16384 tokens."""
    d = workloads.NonCausalReluD128(DEV)
    print("workload noncausal_relu_d128", tuple(d.q.shape), "lengths", d.lengths.tolist(), flush=True)
    d.step()
    torch.cuda.synchronize()
    valid = d.mask.bool()
    # every masked query row is exactly zero
    assert torch.count_nonzero(d.out[~valid]) == 0
    assert torch.isfinite(d.out.float()).all()
    yo, _, _ = oracle.noncausal(f64(d.q), f64(d.k), f64(d.v), d.mask.cpu().numpy(), "relu", True, 1e-6)
    print("out err %.3e worst unit %.3e" % _per_unit_check(d.out, yo, 2e-2, "out", (0, 2)))


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
    assert torch.isfinite(y_chunked.float()).all() and torch.isfinite(d.out_d.float()).all()
    gap, e_cf = _gpu_compare(y_chunked, y_full)
    print("chunked vs full, all units: max abs %.3e, floored rel %.3e" % (gap, e_cf), flush=True)
    assert e_cf <= 2e-2
    # 16 whole batch rows (512 units) against the oracle over all 4096 + 512 tokens:
    # the prefill from a zero state, then the decode tokens from the oracle's state
    rows = _rows(d.B, 16, 4)
    print("oracle rows", rows, flush=True)
    ri = torch.tensor(rows, device=DEV)
    T = d.T
    qr, kr, vr = (f64(t.index_select(0, ri)) for t in (q, k, v))
    yo1, So4, Zo4 = oracle.causal(qr, kr, vr)
    del qr, kr, vr
    qd, kd, vd = (f64(t.index_select(1, ri).transpose(0, 1)) for t in (d.qd, d.kd, d.vd))
    yo2, So, Zo = oracle.causal(qd, kd, vd, S0=So4, Z0=Zo4)
    checks = (
        (y_chunked.index_select(0, ri), yo1, "prefill 4 x 1024", (0, 2)),
        (y_full.index_select(0, ri), yo1, "full 4096 pass", (0, 2)),
        (S_full.index_select(0, ri), So4, "S after 4096", (0, 1)),
        (Z_full.index_select(0, ri), Zo4, "Z after 4096", (0, 1)),
        (d.out_d.index_select(1, ri).transpose(0, 1), yo2, "512 decode outputs", (0, 2)),
        (S_stream.index_select(0, ri), So, "S after 4608", (0, 1)),
        (Z_stream.index_select(0, ri), Zo, "Z after 4608", (0, 1)),
    )
    for x, y, what, ax in checks:
        print(what, "err %.3e worst unit %.3e" % _per_unit_check(x, y, 2e-2, what, ax), flush=True)


def _gated_units_check(d, rule, decay, beta=None, past=None):
    """Every (batch, kv head) unit of a packed gated / delta workload."""
    oo, po = oracle.la_op(f64(d.q), f64(d.k), f64(d.v), d.Hq, d.Hkv, rule, decay=f64(decay),
                          beta=None if beta is None else f64(beta),
                          past_state=None if past is None else f64(past), scale=d.scale)
    G, D = d.Hq // d.Hkv, d.D
    B, T = oo.shape[0], oo.shape[1]
    # out as (B, T, Hkv, G*D): a unit is (b, kv head)
    out = f64(d.out).reshape(B, T, d.Hkv, G * D)
    e1 = _per_unit_check(out, oo.reshape(B, T, d.Hkv, G * D), 2e-2, "out", (0, 2))
    e2 = _per_unit_check(d.present, po, 2e-2, "present", (0, 1))
    print("out err %.3e worst unit %.3e" % e1, "present err %.3e worst unit %.3e" % e2)


def test_gated_gqa_d128_full():
    """All 16 (batch, kv head) units over all 32768 tokens."""
    d = workloads.GatedGqaD128(DEV)
    print("workload gated_gqa_d128", tuple(d.q.shape), "workspace", d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    _gated_units_check(d, "gated", d.g)


def _step_workload_check(d, rule, beta=None):
    """A decode workload of one-token in-place steps (inputs stored step-major,
    (T, B, ...)): every (batch, kv head) unit against one oracle run over the
    tokens from the same past state."""
    past = d.state.clone()
    print("workload", d.name, (d.B, d.T, d.Hq * d.D), "state", tuple(d.state.shape), flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all() and torch.isfinite(d.state).all()
    tb = lambda t: f64(t.transpose(0, 1))
    oo, po = oracle.la_op(tb(d.q), tb(d.k), tb(d.v), d.Hq, d.Hkv, rule, decay=tb(d.g),
                          beta=None if beta is None else tb(beta), past_state=f64(past), scale=d.scale)
    G, D = d.Hq // d.Hkv, d.D
    B, T = oo.shape[0], oo.shape[1]
    out = tb(d.out).reshape(B, T, d.Hkv, G * D)
    e1 = _per_unit_check(out, oo.reshape(B, T, d.Hkv, G * D), 2e-2, "out", (0, 2))
    e2 = _per_unit_check(d.state, po, 2e-2, "state", (0, 1))
    print("out err %.3e worst unit %.3e" % e1, "state err %.3e worst unit %.3e" % e2)


def test_gated_step_d128_full():
    """The gated decode workload: 64 one-token steps of B=256 sequences, in place;
    all 2048 (batch, kv head) units."""
    _step_workload_check(workloads.GatedStepD128(DEV), "gated")


def test_delta_step_d128_full():
    """The gated delta decode workload: 64 one-token steps of B=256 sequences,
    in place, beta per kv head; all 2048 (batch, kv head) units."""
    d = workloads.DeltaStepD128(DEV)
    _step_workload_check(d, "gated_delta", beta=d.beta)


def test_gated_perdim_d128_full():
    """The per-key-dim decay at the GQA workload's sizes (split sequences): all
    16 (batch, kv head) units over all 32768 tokens."""
    d = workloads.GatedPerdimD128(DEV)
    print("workload gated_perdim_d128", tuple(d.q.shape), "decay", tuple(d.g.shape), "workspace",
          d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    _gated_units_check(d, "gated", d.g)


def test_gated_delta_d128_full():
    """The gated delta rule at B=32 T=4096 Hq=32 Hkv=8 D=128: all 256 (batch,
    kv head) units over all 4096 tokens."""
    d = workloads.GatedDeltaD128(DEV)
    print("workload gated_delta_d128", tuple(d.q.shape), flush=True)
    d.step()
    torch.cuda.synchronize()
    assert torch.isfinite(d.out.float()).all()
    _gated_units_check(d, "gated_delta", d.g, beta=d.beta)


def test_backward_bf16_d64_full():
    """The backward workload (B=8 H=16 T=2048 D=64 bf16): all 128 (batch, head)
    units against the oracle backward over all 2048 tokens."""
    d = workloads.BackwardBf16D64(DEV)
    print("workload backward_bf16_d64", tuple(d.q.shape), "workspace", d.ws_bytes, flush=True)
    d.step()
    torch.cuda.synchronize()
    for t in (d.dq, d.dk, d.dv):
        assert torch.isfinite(t.float()).all()
    oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(d.q), f64(d.k), f64(d.v), f64(d.dy))
    for x, y, w, ax in ((d.dq, oq, "dq", (0, 2)), (d.dk, ok_, "dk", (0, 2)), (d.dv, ov, "dv", (0, 2)),
                        (d.dS0, oS, "dS0", (0, 1)), (d.dZ0, oZ, "dZ0", (0, 1))):
        print(w, "err %.3e worst unit %.3e" % _per_unit_check(x, y, 2e-2, w, ax))
