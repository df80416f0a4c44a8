"""Edge cases on the GPU, through the C ABI:

* near-zero denominators (the Keras proposal's "Test Plan" lists them under
  numerical stability): relu(x)+eps with every query and/or key entry <= 0,
  so that phi is eps in every dimension, and elu(x)+1 at strongly negative
  inputs, where phi(q).Z falls below eps; causal prefill, non-causal and the
  T=1 step, every dtype, against the fp64 oracle;
* guard regions: every output, state and workspace buffer sits inside a larger
  allocation whose head and tail are filled with NaN (or 0xFF bytes); after the
  call the guards must be untouched, for every entry point and path (single
  pass, split sequence, non-causal, step, gated per head / per dim, delta,
  backward);
* the binding's buffer checks: strided or wrongly typed state buffers are
  rejected or copied, never read as raw float32 or written through a copy.
"""
import pytest
import torch

import oracle
import synth
import kernelized_linear_attention_chunked_amd as la
from _util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = [torch.float32, torch.bfloat16, torch.float16]
DT_IDS = ["f32", "bf16", "f16"]


# --------------------------------------------------------- near-zero denominators
def _nz_inputs(B, T, H, D, dtype, seed, case):
    """q, k, v for one near-zero-denominator case."""
    q, k, v = synth.qkv(B, T, H, D, torch.float32, DEV, seed, 1.0, 1.0, 1.0)
    if case == "relu_k_nonpos":
        k = -k.abs()
    elif case == "relu_q_nonpos":
        q = -q.abs()
    elif case == "relu_both_nonpos":
        q, k = -q.abs(), -k.abs()
    elif case == "elu_very_negative":
        # phi = exp(x) with x ~ N(-10, 1): phi(q).phi(k) summed over D is ~1e-7,
        # below eps = 1e-6, so eps dominates every denominator
        q, k = q - 10.0, k - 10.0
    else:
        raise ValueError(case)
    return q.to(dtype), k.to(dtype), v.to(dtype)


NZ_CASES = ["relu_k_nonpos", "relu_q_nonpos", "relu_both_nonpos", "elu_very_negative"]


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("case", NZ_CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_near_zero_denominator_causal_and_step(dtype, case, D):
    B, T, H = 2, 150, 3
    fm = "elu_plus_one" if case.startswith("elu") else "relu"
    q, k, v = _nz_inputs(B, T + 1, H, D, dtype, 40 + D, case)
    y, state = la.la_forward(q[:, :T], k[:, :T], v[:, :T], causal=True, feature_map=fm, return_state=True)
    ys, state = la.la_step(q[:, T], k[:, T], v[:, T], state, feature_map=fm)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), feature_map=fm)
    tol = TOL[dtype]
    assert_close(y, yo[:, :T], tol, "prefill")
    assert_close(ys, yo[:, T], tol, "step")
    assert_close(state[0], So, tol, "S")
    assert_close(state[1], Zo, tol, "Z")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("case", NZ_CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_near_zero_denominator_noncausal(dtype, case, D):
    B, T, H = 2, 230, 2
    fm = "elu_plus_one" if case.startswith("elu") else "relu"
    q, k, v = _nz_inputs(B, T, H, D, dtype, 50 + D, case)
    mask, _ = synth.right_padding_mask(B, T, DEV, 50 + D, lo=100, hi=T)
    y = la.la_forward(q, k, v, mask=mask, causal=False, feature_map=fm)
    torch.cuda.synchronize()
    yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), mask.cpu().numpy(), fm, True, 1e-6)
    assert_close(y, yo, TOL[dtype], "out")
    assert torch.all(y[~mask] == 0)


# ------------------------------------------------------------------ guard regions
GUARD = 256  # elements of guard before and after each buffer (keeps 16-byte alignment)


class Guarded:
    """A buffer of ``shape`` inside a larger allocation with NaN guards (0xFF
    bytes for integer buffers) before and after it."""

    def __init__(self, shape, dtype):
        n = 1
        for s in shape:
            n *= int(s)
        self.n = n
        self.full = torch.empty(n + 2 * GUARD, dtype=dtype, device=DEV)
        if dtype.is_floating_point:
            self.full.fill_(float("nan"))
        else:
            self.full.view(torch.uint8).fill_(0xFF)
        self.ref = self.full.clone()
        self.t = self.full[GUARD:GUARD + n].view(shape)

    def check(self, what):
        head = self.full[:GUARD].view(torch.uint8)
        tail = self.full[GUARD + self.n:].view(torch.uint8)
        assert torch.equal(head, self.ref[:GUARD].view(torch.uint8)), "%s: head guard written" % what
        assert torch.equal(tail, self.ref[GUARD + self.n:].view(torch.uint8)), "%s: tail guard written" % what


def _ws(nbytes):
    return Guarded((max(nbytes, 16),), torch.uint8)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("shape", [(2, 200, 3, 64), (1, 1500, 2, 128), (64, 70, 8, 32)],
                         ids=["split", "split_d128", "single_pass"])
def test_guards_forward_causal(dtype, shape):
    B, T, H, D = shape
    q, k, v = synth.qkv(B, T, H, D, dtype, DEV, 60)
    out = Guarded((B, T, H, D), dtype)
    s_kv, s_k = Guarded((B, H, D, D), torch.float32), Guarded((B, H, D), torch.float32)
    ws = _ws(la.la_workspace_size(B, T, H, D, D, dtype, True))
    y = la.la_forward(q, k, v, causal=True, out=out.t, state_out=(s_kv.t, s_k.t), workspace=ws.t)
    torch.cuda.synchronize()
    for g, n in ((out, "out"), (s_kv, "S"), (s_k, "Z"), (ws, "workspace")):
        g.check(n)
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    assert_close(y, yo, TOL[dtype], "out")
    assert_close(s_kv.t, So, TOL[dtype], "S")
    # in place over a guarded state, then a step over it
    la.la_initial_state(B, H, D, D, out=(s_kv.t, s_k.t))
    la.la_forward(q, k, v, causal=True, state=(s_kv.t, s_k.t), state_out=(s_kv.t, s_k.t),
                  out=out.t, workspace=ws.t)
    yd = Guarded((B, H, D), dtype)
    la.la_step(q[:, -1], k[:, -1], v[:, -1], (s_kv.t, s_k.t), out=yd.t)
    torch.cuda.synchronize()
    for g, n in ((out, "out"), (s_kv, "S"), (s_k, "Z"), (ws, "workspace"), (yd, "step out")):
        g.check(n)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [64, 128])
def test_guards_forward_noncausal(dtype, D):
    B, T, H = 2, 700, 3
    q, k, v = synth.qkv(B, T, H, D, dtype, DEV, 61)
    mask, _ = synth.right_padding_mask(B, T, DEV, 61)
    out = Guarded((B, T, H, D), dtype)
    ws = _ws(la.la_workspace_size(B, T, H, D, D, dtype, False))
    la.la_forward(q, k, v, mask=mask, causal=False, feature_map="relu", out=out.t, workspace=ws.t)
    torch.cuda.synchronize()
    out.check("out")
    ws.check("workspace")
    yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), mask.cpu().numpy(), "relu", True, 1e-6)
    assert_close(out.t, yo, TOL[dtype], "out")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("rule", ["gated", "gated_perdim", "delta", "gated_delta"])
@pytest.mark.parametrize("T", [1, 300, 2048])
def test_guards_gated_and_delta(dtype, rule, T):
    B, Hq, Hkv, D = 1, 4, 2, 64
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, 62, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, 62, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, 62, "v")
    g = None
    if rule in ("gated", "gated_delta"):
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, 62)
    elif rule == "gated_perdim":
        g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, 62)
    out = Guarded((B, T, Hq * D), dtype)
    pres = Guarded((B, Hkv, D, D), torch.float32)
    if rule.endswith("delta"):
        beta = torch.sigmoid(synth.normal((B, T, Hkv), 1.0, torch.float32, DEV, 62, "beta")).to(dtype)
        la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, out=out.t, present_state=pres.t)
        guards = ((out, "out"), (pres, "present"))
    else:
        beta = None
        ws = _ws(la.la_gated_workspace_size(B, T, Hq, Hkv, D, D, dtype, rule == "gated_perdim"))
        la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, out=out.t, present_state=pres.t, workspace=ws.t)
        guards = ((out, "out"), (pres, "present"), (ws, "workspace"))
    torch.cuda.synchronize()
    for gd, n in guards:
        gd.check(n)
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated" if rule == "gated_perdim" else rule,
                          decay=None if g is None else f64(g), beta=None if beta is None else f64(beta))
    assert_close(out.t, oo, TOL[dtype], "out")
    assert_close(pres.t, po, TOL[dtype], "present")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_guards_gated_step(dtype):
    B, Hq, Hkv, D = 3, 8, 2, 128
    q = synth.normal((B, Hq * D), 1.0, dtype, DEV, 63, "q")
    k = synth.l2_normalized((B, Hkv, D), dtype, DEV, 63, "k").reshape(B, Hkv * D)
    v = synth.normal((B, Hkv * D), 1.0, dtype, DEV, 63, "v")
    g = synth.logsigmoid_decay((B, Hkv), dtype, DEV, 63)
    out = Guarded((B, Hq * D), dtype)
    st = Guarded((B, Hkv, D, D), torch.float32)
    st.t.normal_()
    past = st.t.clone()
    la.la_gated_step(q, k, v, Hq, Hkv, decay=g, past_state=st.t, in_place=True, out=out.t)
    torch.cuda.synchronize()
    out.check("out")
    st.check("state")
    oo, po = oracle.la_op(f64(q)[:, None], f64(k)[:, None], f64(v)[:, None], Hq, Hkv, "gated",
                          decay=f64(g)[:, None], past_state=f64(past))
    assert_close(out.t, oo[:, 0], TOL[dtype], "out")
    assert_close(st.t, po, TOL[dtype], "state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_guards_backward(dtype):
    """la_backward through the C ABI with guarded gradient buffers and workspace."""
    import ctypes
    B, T, H, D = 2, 300, 3, 64
    q, k, v = synth.qkv(B, T, H, D, dtype, DEV, 64)
    dy = synth.normal((B, T, H, D), 1.0, dtype, DEV, 64, "dy")
    lib = la.load_library()
    n = ctypes.c_size_t(0)
    code = {torch.float32: 0, torch.bfloat16: 1}[dtype]
    assert lib.la_backward_workspace_size(B, T, H, D, D, code, 1, ctypes.byref(n)) == 0
    grads = [Guarded((B, T, H, D), dtype) for _ in range(3)]
    dS0, dZ0 = Guarded((B, H, D, D), torch.float32), Guarded((B, H, D), torch.float32)
    ws = _ws(n.value)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.la_backward(P(q), P(k), P(v), None, None, None, P(dy), None, None, 0, 1, ctypes.c_float(1e-6),
                         P(grads[0].t), P(grads[1].t), P(grads[2].t), P(dS0.t), P(dZ0.t), B, T, H, D, D, code,
                         P(ws.t), n.value, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.la_last_error_message()
    torch.cuda.synchronize()
    for gd, nm in zip(grads + [dS0, dZ0, ws], ("dq", "dk", "dv", "dS0", "dZ0", "workspace")):
        gd.check(nm)
    oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(q), f64(k), f64(v), f64(dy))
    for gd, o, nm in zip(grads + [dS0, dZ0], (oq, ok_, ov, oS, oZ), ("dq", "dk", "dv", "dS0", "dZ0")):
        assert_close(gd.t, o, TOL[dtype], nm)


# ------------------------------------------------------------- binding buffer checks
def test_backward_strided_state_and_dstate():
    """Non-contiguous state and dstate: the binding's contiguous copies stay
    alive until the call, so the result equals the contiguous call's."""
    B, T, H, D = 2, 200, 3, 64
    q, k, v = synth.qkv(B, T, H, D, torch.bfloat16, DEV, 65)
    dy = synth.normal((B, T, H, D), 1.0, torch.bfloat16, DEV, 65, "dy")
    S0 = torch.randn((B, H, D, D), device=DEV) * 0.3
    Z0 = torch.rand((B, H, D), device=DEV) + 0.5
    dS = torch.randn((B, H, D, D), device=DEV)
    dZ = torch.randn((B, H, D), device=DEV)
    ref = la.la_backward(q, k, v, dy, state=(S0, Z0), dstate=(dS, dZ))
    # transposed views of the same values (same shape, other strides)
    S0t = S0.transpose(2, 3).contiguous().transpose(2, 3)
    dSt = dS.transpose(2, 3).contiguous().transpose(2, 3)
    assert not S0t.is_contiguous() and not dSt.is_contiguous()
    got = la.la_backward(q, k, v, dy, state=(S0t, Z0), dstate=(dSt, dZ))
    torch.cuda.synchronize()
    for a, b in zip(ref[:3] + ref[3], got[:3] + got[3]):
        assert torch.equal(a, b)


def test_binding_rejects_bad_state_buffers():
    B, T, H, D = 2, 64, 2, 64
    q, k, v = synth.qkv(B, T, H, D, torch.bfloat16, DEV, 66)
    kv, z = la.la_initial_state(B, H, D, D)
    with pytest.raises(ValueError):   # a bf16 state would be read as raw float32
        la.la_forward(q, k, v, state=(kv.to(torch.bfloat16), z), return_state=True)
    with pytest.raises(ValueError):   # a strided in-place state would update a copy
        la.la_step(q[:, 0], k[:, 0], v[:, 0], (kv.transpose(2, 3), z))
    with pytest.raises(ValueError):   # wrong shape
        la.la_forward(q, k, v, state=(kv[:, :, :32], z), return_state=True)
    with pytest.raises(ValueError):
        la.la_forward(q, k, v, out=torch.empty((B, T, H, D), dtype=torch.float32, device=DEV))
    Hq, Hkv = 4, 2
    qg = synth.normal((1, 1, Hq * D), 1.0, torch.bfloat16, DEV, 66, "q")
    kg = synth.normal((1, 1, Hkv * D), 1.0, torch.bfloat16, DEV, 66, "k")
    vg = synth.normal((1, 1, Hkv * D), 1.0, torch.bfloat16, DEV, 66, "v")
    past = torch.zeros((1, Hkv, D, D), device=DEV).transpose(2, 3)
    with pytest.raises(ValueError):
        la.la_gated_step(qg, kg, vg, Hq, Hkv, past_state=past, in_place=True)
    # as an input a strided past state is fine (copied, held for the call)
    out, pres = la.la_gated_step(qg, kg, vg, Hq, Hkv, past_state=past, in_place=False)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(qg), f64(kg), f64(vg), Hq, Hkv, "linear", past_state=f64(past))
    assert_close(out, oo, 2e-2, "out")
    assert_close(pres, po, 2e-2, "present")
