"""GPU parity of the HIP library against the fp64 oracle, at small sizes that
still span several 64-token chunks, a ragged tail, split sequences and the
single-pass path.  Every call goes through the C ABI (via the ctypes binding).

Tolerance: floored relative error (tests/_util.py) <= 1e-4 for fp32 inputs,
<= 2e-2 for bf16 and fp16 inputs with fp32 state."""
import json
import os

import numpy as np
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
FMS = ["elu_plus_one", "relu"]


def _inputs(B, T, H, D, dtype, seed, qk_std=0.5):
    return synth.qkv(B, T, H, D, dtype, DEV, seed, qk_std, qk_std, 1.0)


def _state(B, H, D, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    S = torch.randn((B, H, D, D), generator=g) * 0.5
    Z = torch.rand((B, H, D), generator=g) * 4 + 0.5
    return S.to(DEV), Z.to(DEV)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("fm", FMS)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_causal_small(dtype, D, fm, norm):
    B, T, H = 2, 200, 3                 # 4 chunks, ragged tail of 8 tokens, split sequence
    seed = D + 7 * norm + 13 * (fm == "relu") + 31 * (dtype == torch.bfloat16)
    q, k, v = _inputs(B, T, H, D, dtype, seed)
    mask = synth.random_mask(B, T, 0.85, DEV, seed)
    S0, Z0 = _state(B, H, D, seed)
    state = (S0, Z0 if norm else None)
    y, (S, Z) = la.la_forward(q, k, v, mask=mask, state=state, causal=True, feature_map=fm,
                              use_normalizer=norm, eps=1e-6, return_state=True)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), f64(mask) > 0, f64(S0),
                               f64(Z0) if norm else None, fm, norm, 1e-6)
    tol = TOL[dtype]
    assert_close(y, yo, tol, "out")
    assert_close(S, So, tol, "S")
    if norm:
        assert_close(Z, Zo, tol, "Z")
    # masked queries are exactly zero
    m = mask.cpu().numpy()
    assert np.all(f64(y)[~m] == 0.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_causal_split_state_in_place(dtype, D):
    """A split sequence (6 units of 16 chunks) whose state is updated in place:
    every segment starts from the initial state before the last one writes the
    final state over it."""
    B, T, H = 2, 1000, 3
    q, k, v = _inputs(B, T, H, D, dtype, 4400 + D)
    S0, Z0 = _state(B, H, D, 4400 + D)
    S, Z = S0.clone(), Z0.clone()
    y = la.la_forward(q, k, v, state=(S, Z), causal=True, state_out=(S, Z))
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), None, f64(S0), f64(Z0))
    assert_close(y, yo, TOL[dtype], "out")
    assert_close(S, So, TOL[dtype], "S")
    assert_close(Z, Zo, TOL[dtype], "Z")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [64, 128])
def test_causal_single_pass_path(dtype, D):
    # 512 (batch, head) units: one pass, state carried across all chunks in a workgroup
    B, T, H = 4, 130, 128
    q, k, v = _inputs(B, T, H, D, dtype, 99 + D)
    y, (S, Z) = la.la_forward(q, k, v, causal=True, return_state=True)
    torch.cuda.synchronize()
    idx = [(0, 0), (1, 77), (3, 127), (2, 5)]
    for b, h in idx:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        yo, So, Zo = oracle.causal(f64(q[sl]), f64(k[sl]), f64(v[sl]))
        assert_close(y[sl], yo, TOL[dtype], "out %d,%d" % (b, h))
        assert_close(S[b:b + 1, h:h + 1], So, TOL[dtype], "S")
        assert_close(Z[b:b + 1, h:h + 1], Zo, TOL[dtype], "Z")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 1000])
def test_causal_lengths(T):
    B, H, D = 1, 2, 64
    q, k, v = _inputs(B, T, H, D, torch.bfloat16, T)
    y, (S, Z) = la.la_forward(q, k, v, causal=True, return_state=True)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    assert_close(y, yo, 2e-2, "out")
    assert_close(S, So, 2e-2, "S")
    assert_close(Z, Zo, 2e-2, "Z")


def test_causal_zero_length_passes_state_through():
    B, H, D = 2, 3, 32
    q = torch.empty((B, 0, H, D), device=DEV)
    S0, Z0 = _state(B, H, D, 5)
    y, (S, Z) = la.la_forward(q, q, q, state=(S0, Z0), causal=True, return_state=True)
    torch.cuda.synchronize()
    assert y.shape == (B, 0, H, D)
    assert torch.equal(S, S0) and torch.equal(Z, Z0)
    _, (S, Z) = la.la_forward(q, q, q, causal=True, return_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0 and torch.count_nonzero(Z) == 0


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("fm", FMS)
def test_masked_garbage_does_not_leak(dtype, fm):
    B, T, H, D = 2, 150, 2, 64
    q, k, v = _inputs(B, T, H, D, dtype, 21)
    mask = synth.random_mask(B, T, 0.7, DEV, 21)
    y1, (S1, Z1) = la.la_forward(q, k, v, mask=mask, feature_map=fm, return_state=True)
    qn, kn, vn = q.clone(), k.clone(), v.clone()
    bad = ~mask
    for t in (qn, kn, vn):
        t[bad] = float("nan")
    y2, (S2, Z2) = la.la_forward(qn, kn, vn, mask=mask, feature_map=fm, return_state=True)
    y3 = la.la_forward(qn, kn, vn, mask=mask, feature_map=fm, causal=False)
    y4 = la.la_forward(q, k, v, mask=mask, feature_map=fm, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2) and torch.equal(Z1, Z2)
    assert torch.equal(y3, y4)
    assert torch.all(y2[bad] == 0) and torch.all(y3[bad] == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_fully_masked_chunks(dtype, D, causal):
    # whole 64-token chunks without a valid token are skipped by the kernels: the
    # state passes through them, their outputs are written as zeros (the output
    # buffer starts as NaN) and their inputs (NaN here) are never read
    B, T, H = 2, 330, 2
    q, k, v = _inputs(B, T, H, D, dtype, 500 + D, qk_std=0.5 if causal else 1.0)
    mask = torch.ones((B, T), dtype=torch.bool, device=DEV)
    mask[0, 64:192] = False     # two dead chunks in the middle
    mask[0, 256:] = False       # dead tail
    mask[0, 5] = False          # and a partly masked chunk
    mask[1, 70:] = False        # row 1: chunk 1 partly valid, the rest dead
    qn, kn, vn = q.clone(), k.clone(), v.clone()
    for t in (qn, kn, vn):
        t[~mask] = float("nan")
    out = torch.full((B, T, H, D), float("nan"), dtype=dtype, device=DEV)
    m = mask.cpu().numpy()
    if causal:
        S0, Z0 = _state(B, H, D, 500 + D)
        y, (S, Z) = la.la_forward(qn, kn, vn, mask=mask, state=(S0, Z0), causal=True,
                                  return_state=True, out=out)
        torch.cuda.synchronize()
        yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), m, f64(S0), f64(Z0))
        assert_close(S, So, TOL[dtype], "S")
        assert_close(Z, Zo, TOL[dtype], "Z")
    else:
        y = la.la_forward(qn, kn, vn, mask=mask, causal=False, feature_map="relu", out=out)
        torch.cuda.synchronize()
        yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), m, "relu", True, 1e-6)
    assert torch.all(y[~mask] == 0)
    assert_close(y, yo, TOL[dtype], "out")


def test_all_false_and_all_true_masks():
    B, T, H, D = 2, 100, 2, 32
    q, k, v = _inputs(B, T, H, D, torch.float32, 3)
    S0, Z0 = _state(B, H, D, 3)
    y, (S, Z) = la.la_forward(q, k, v, mask=torch.zeros((B, T), dtype=torch.bool, device=DEV),
                              state=(S0, Z0), return_state=True)
    ya = la.la_forward(q, k, v, mask=torch.ones((B, T), dtype=torch.bool, device=DEV))
    yb = la.la_forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
    assert torch.equal(S, S0) and torch.equal(Z, Z0)
    assert torch.equal(ya, yb)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("fm", FMS)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_noncausal_small(dtype, D, fm, norm):
    B, T, H = 2, 300, 2
    seed = 1000 + D + 7 * norm + 13 * (fm == "relu")
    q, k, v = _inputs(B, T, H, D, dtype, seed, qk_std=1.0)
    mask, _ = synth.right_padding_mask(B, T, DEV, seed, lo=100, hi=T)
    y = la.la_forward(q, k, v, mask=mask, causal=False, feature_map=fm, use_normalizer=norm)
    torch.cuda.synchronize()
    yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), mask.cpu().numpy(), fm, norm, 1e-6)
    assert_close(y, yo, TOL[dtype], "out")
    assert torch.all(y[~mask] == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("fm", FMS)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
@pytest.mark.parametrize("in_place", [True, False], ids=["inplace", "copy"])
def test_decode_step(dtype, D, fm, norm, in_place):
    B, H = 3, 5
    seed = 2000 + D
    q, k, v = _inputs(B, 1, H, D, dtype, seed)
    S0, Z0 = _state(B, H, D, seed)
    mask = torch.tensor([True, False, True], device=DEV)
    s_kv, s_k = S0.clone(), (Z0.clone() if norm else None)
    y, (S, Z) = la.la_step(q, k, v, (s_kv, s_k), mask=mask, feature_map=fm, use_normalizer=norm,
                           in_place=in_place)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), mask.cpu().numpy()[:, None], f64(S0),
                               f64(Z0) if norm else None, fm, norm, 1e-6)
    assert_close(y, yo[:, 0] if y.dim() == 3 else yo, TOL[dtype], "out")
    assert_close(S, So, TOL[dtype], "S")
    if norm:
        assert_close(Z, Zo, TOL[dtype], "Z")
    assert torch.all(y[1] == 0)
    assert torch.equal(S[1], S0[1])
    if in_place:
        assert S.data_ptr() == s_kv.data_ptr()


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_chunked_and_step_equal_full(dtype):
    B, T, H, D = 2, 320, 4, 64
    q, k, v = _inputs(B, T, H, D, dtype, 77)
    y_full, (S_full, Z_full) = la.la_forward(q, k, v, return_state=True)
    state = la.la_initial_state(B, H, D, D)
    ys = []
    for a, b in ((0, 64), (64, 100), (100, 101), (101, 256), (256, 300)):
        y, state = la.la_forward(q[:, a:b], k[:, a:b], v[:, a:b], state=state, return_state=True)
        ys.append(y)
    for t in range(300, T):
        y, state = la.la_step(q[:, t], k[:, t], v[:, t], state)
        ys.append(y[:, None])
    torch.cuda.synchronize()
    y_chunked = torch.cat(ys, 1)
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    tol = TOL[dtype]
    assert_close(y_full, yo, tol, "full")
    assert_close(y_chunked, yo, tol, "chunked+steps")
    assert_close(state[0], So, tol, "S chunked")
    assert_close(state[1], Zo, tol, "Z chunked")
    assert_close(S_full, So, tol, "S full")


def test_initial_state_is_zero():
    kv, k = la.la_initial_state(3, 4, 64, 64)
    kv2, k2 = la.la_initial_state(3, 4, 64, 64, use_normalizer=False)
    torch.cuda.synchronize()
    assert kv.shape == (3, 4, 64, 64) and k.shape == (3, 4, 64) and k2 is None
    assert torch.count_nonzero(kv) == 0 and torch.count_nonzero(k) == 0
    assert torch.count_nonzero(kv2) == 0


# ------------------------------------------------------------------ gated / GQA
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "linear"])
def test_gated_small(dtype, D, G, gated):
    B, T, Hkv = 2, 190, 2
    Hq = Hkv * G
    seed = 3000 + D + G + 50 * gated
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=1.0) if gated else None
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated" if gated else "linear",
                          past_state=f64(past), decay=None if g is None else f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


def test_gated_present_aliases_past():
    B, T, Hkv, G, D = 1, 300, 2, 4, 64
    Hq = Hkv * G
    q = synth.normal((B, T, Hq * D), 1.0, torch.bfloat16, DEV, 5, "q")
    k = synth.l2_normalized((B, T, Hkv, D), torch.bfloat16, DEV, 5, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, torch.bfloat16, DEV, 5, "v")
    g = synth.logsigmoid_decay((B, T, Hkv), torch.bfloat16, DEV, 5)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 5, "past")
    out_a, pres_a = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past.clone())
    buf = past.clone()
    out_b, pres_b = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=buf, present_state=buf)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pres_a, pres_b)


# ------------------------------------------------------------- causal backward
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("fm", FMS)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_backward_small(dtype, D, fm, norm):
    B, T, H = 2, 150, 2
    seed = 7000 + D + 7 * norm + 13 * (fm == "relu")
    q, k, v = _inputs(B, T, H, D, dtype, seed)
    dy = synth.normal((B, T, H, D), 1.0, dtype, DEV, seed, "dy")
    dq, dk, dv, (dS0, dZ0) = la.la_backward(q, k, v, dy, feature_map=fm, use_normalizer=norm)
    torch.cuda.synchronize()
    oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(q), f64(k), f64(v), f64(dy), feature_map=fm,
                                                 use_normalizer=norm)
    tol = TOL[dtype]
    assert_close(dq, oq, tol, "dq")
    assert_close(dk, ok_, tol, "dk")
    assert_close(dv, ov, tol, "dv")
    assert_close(dS0, oS, tol, "dS0")
    if norm:
        assert_close(dZ0, oZ, tol, "dZ0")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("fm", FMS)
def test_backward_state_and_mask(dtype, fm):
    """An initial state, a gradient of the final state, a random mask."""
    B, T, H, D = 2, 200, 3, 64
    q, k, v = _inputs(B, T, H, D, dtype, 91)
    dy = synth.normal((B, T, H, D), 1.0, dtype, DEV, 91, "dy")
    S0, Z0 = _state(B, H, D, 91)
    gS = synth.normal((B, H, D, D), 0.2, torch.float32, DEV, 91, "gS")
    gZ = synth.normal((B, H, D), 0.2, torch.float32, DEV, 91, "gZ")
    mask = synth.random_mask(B, T, 0.8, DEV, 91)
    dq, dk, dv, (dS0, dZ0) = la.la_backward(q, k, v, dy, mask=mask, state=(S0, Z0), dstate=(gS, gZ),
                                            feature_map=fm)
    torch.cuda.synchronize()
    oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(q), f64(k), f64(v), f64(dy), f64(mask) > 0, f64(S0),
                                                 f64(Z0), f64(gS), f64(gZ), feature_map=fm)
    tol = TOL[dtype]
    for x, y, what in ((dq, oq, "dq"), (dk, ok_, "dk"), (dv, ov, "dv"), (dS0, oS, "dS0"), (dZ0, oZ, "dZ0")):
        assert_close(x, y, tol, what)
    invalid = ~mask.bool()
    assert not dq[invalid].float().abs().sum() and not dk[invalid].float().abs().sum()
    assert not dv[invalid].float().abs().sum()


def test_backward_split_sequence():
    """Few units and a long sequence: the recurrences run split over T."""
    B, T, H, D = 1, 3000, 1, 64
    q, k, v = _inputs(B, T, H, D, torch.bfloat16, 92)
    dy = synth.normal((B, T, H, D), 1.0, torch.bfloat16, DEV, 92, "dy")
    dq, dk, dv, (dS0, dZ0) = la.la_backward(q, k, v, dy)
    torch.cuda.synchronize()
    oq, ok_, ov, oS, oZ = oracle.causal_backward(f64(q), f64(k), f64(v), f64(dy))
    for x, y, what in ((dq, oq, "dq"), (dk, ok_, "dk"), (dv, ov, "dv"), (dS0, oS, "dS0"), (dZ0, oZ, "dZ0")):
        assert_close(x, y, 2e-2, what)


# --------------------------------------------------- per-key-dim decay (GLA form)
def _pd_inputs(B, T, Hq, Hkv, D, dtype, seed, mean=1.0):
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=mean)
    return q, k, v, g


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gated_perdim_small(dtype, D, G):
    B, T, Hkv = 2, 190, 2
    Hq = Hkv * G
    q, k, v, g = _pd_inputs(B, T, Hq, Hkv, D, dtype, 5000 + D + G)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 5000 + D + G, "past")
    # (fp32 at head size 128 runs token by token)
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", past_state=f64(past), decay=f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_gated_perdim_split_sequence(dtype):
    """Few units and a long sequence: segments in state mode, the per-dim affine
    prefix, then the output pass."""
    B, T, Hkv, G, D = 1, 3000, 1, 2, 64
    Hq = Hkv * G
    q, k, v, g = _pd_inputs(B, T, Hq, Hkv, D, dtype, 71)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 71, "past")
    assert la.la_gated_workspace_size(B, T, Hq, Hkv, D, D, dtype, True) > 0
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", past_state=f64(past), decay=f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gated_perdim_strong_decay(dtype):
    """Decays of about -1.3 per token and dim (some near -4): about -40 summed
    over a 32-token block, well inside the keys' rescaling range."""
    B, T, Hkv, G, D = 2, 200, 2, 2, 64
    Hq = Hkv * G
    q, k, v, g = _pd_inputs(B, T, Hq, Hkv, D, dtype, 72, mean=-1.0)
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", decay=f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_gated_perdim_step(dtype, D, G):
    B, Hkv = 3, 2
    Hq = Hkv * G
    q, k, v, g = _pd_inputs(B, 1, Hq, Hkv, D, dtype, 5100 + D + G)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 5100 + D + G, "past")
    ref = f64(past)
    out, present = la.la_gated_step(q, k, v, Hq, Hkv, decay=g, past_state=past, in_place=True)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", past_state=ref, decay=f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_gated_perdim_prefill_then_steps(dtype):
    B, T0, N, Hkv, G, D = 2, 70, 5, 2, 2, 64
    Hq, T = Hkv * G, T0 + N
    q, k, v, g = _pd_inputs(B, T, Hq, Hkv, D, dtype, 73)
    y0, state = la.la_gated_forward(q[:, :T0], k[:, :T0], v[:, :T0], Hq, Hkv, decay=g[:, :T0])
    ys = [y0]
    for t in range(T0, T):
        y, state = la.la_gated_step(q[:, t], k[:, t], v[:, t], Hq, Hkv, decay=g[:, t],
                                    past_state=state, in_place=True)
        ys.append(y[:, None])
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", decay=f64(g))
    assert_close(torch.cat(ys, 1), oo, TOL[dtype], "outputs")
    assert_close(state, po, TOL[dtype], "state")


# ------------------------------------------------------- delta / gated-delta rules
def _beta(shape, dtype, seed):
    x = synth.normal(shape, 1.0, torch.float32, DEV, seed, "beta")
    return torch.sigmoid(x).to(dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("kind", ["delta", "gated_head", "gated_dim"])
def test_delta_small(dtype, D, G, kind):
    B, T, Hkv = 2, 150, 2
    Hq = Hkv * G
    seed = 6000 + D + G + 7 * len(kind)
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    beta = _beta((B, T, Hkv), dtype, seed)
    g = None
    if kind == "gated_head":
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=1.0)
    elif kind == "gated_dim":
        g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=1.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    # (fp32 at head size 128 with a per-dim decay runs token by token)
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "delta" if g is None else "gated_delta",
                          past_state=f64(past), decay=None if g is None else f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("kind", ["delta", "gated_head", "gated_dim"])
def test_delta_step(dtype, D, G, kind):
    """T = 1 runs the streaming step kernel (fp32 at head size 128 included):
    one token against the oracle; the per-head case runs in place and the
    plain delta rule with beta shared by the kv heads."""
    B, Hkv = 3, 2
    Hq = Hkv * G
    seed = 7000 + D + G + 7 * len(kind)
    q = synth.normal((B, 1, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, 1, Hkv, D), dtype, DEV, seed, "k").reshape(B, 1, Hkv * D)
    v = synth.normal((B, 1, Hkv * D), 1.0, dtype, DEV, seed, "v")
    beta = _beta((B, 1, 1 if kind == "delta" else Hkv), dtype, seed)
    g = None
    if kind == "gated_head":
        g = synth.logsigmoid_decay((B, 1, Hkv), dtype, DEV, seed, mean=1.0)
    elif kind == "gated_dim":
        g = synth.logsigmoid_decay((B, 1, Hkv * D), dtype, DEV, seed, mean=1.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    ref_past = f64(past)
    if kind == "gated_head":
        state = past.clone()
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=state,
                                           present_state=state)
        assert present.data_ptr() == state.data_ptr()
    else:
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "delta" if g is None else "gated_delta",
                          past_state=ref_past, decay=None if g is None else f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("kind", ["delta", "gated_head", "gated_dim"])
def test_delta_prefill_then_steps(dtype, kind):
    """A 100-token call followed by 20 T = 1 steps, each from the state the last
    call returned, against the oracle over the whole 120 tokens."""
    B, T0, T1, Hkv, G, D = 2, 100, 20, 2, 2, 64
    Hq, T = Hkv * G, T0 + T1
    seed = 7300 + len(kind)
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    beta = _beta((B, T, Hkv), dtype, seed)
    g = None
    if kind == "gated_head":
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=1.0)
    elif kind == "gated_dim":
        g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=1.0)
    sl = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
    out0, state = la.la_delta_forward(sl(q, 0, T0), sl(k, 0, T0), sl(v, 0, T0), Hq, Hkv, sl(beta, 0, T0),
                                      decay=sl(g, 0, T0))
    outs = [out0]
    for t in range(T0, T):
        o, state = la.la_delta_forward(sl(q, t, t + 1), sl(k, t, t + 1), sl(v, t, t + 1), Hq, Hkv,
                                       sl(beta, t, t + 1), decay=sl(g, t, t + 1), past_state=state)
        outs.append(o)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "delta" if g is None else "gated_delta",
                          decay=None if g is None else f64(g), beta=f64(beta))
    assert_close(torch.cat(outs, dim=1), oo, TOL[dtype], "out")
    assert_close(state, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("G", [1, 4])
def test_delta_strong_head_decay(dtype, G):
    """Per-head decays of about -20 per token: every decay factor past the
    diagonal would overflow, and the state forgets within a few tokens.  fp32
    and bf16 inputs apply the factors after the products and take any
    strength; fp16 inputs rescale the keys per 32-token block and get about
    -1.3 per token, inside that range."""
    B, T, Hkv, D = 1, 200, 2, 64
    Hq = Hkv * G
    seed = 6500 + G
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    beta = _beta((B, T, Hkv), dtype, seed)
    g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=-1.0 if dtype == torch.float16 else -20.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(present).all()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated_delta", past_state=f64(past),
                          decay=f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("G", [2, 8])
@pytest.mark.parametrize("kind", ["delta", "gated_head", "gated_head_strong"])
def test_delta_f32_d128(G, kind):
    """fp32 inputs at head size 128 (no decay or a per-head one) over several
    chunks and a ragged tail, the two wider GQA groups; the strong case has
    per-head decays of about -20 per token, which fp32 takes at any strength."""
    dtype, D, B, T, Hkv = torch.float32, 128, 1, 213, 2
    Hq = Hkv * G
    seed = 6600 + G + 7 * len(kind)
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    beta = _beta((B, T, Hkv), dtype, seed)
    g = None
    if kind != "delta":
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=-20.0 if kind.endswith("strong") else 1.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "delta" if g is None else "gated_delta",
                          past_state=f64(past), decay=None if g is None else f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("G,in_place", [(1, True), (4, True), (8, False), (16, True), (16, False)])
@pytest.mark.parametrize("rule", ["gated", "gated_delta"])
@pytest.mark.parametrize("mean", [1.0, -20.0], ids=["mild", "strong"])
def test_perdim_f32_d128_token_by_token(G, in_place, rule, mean):
    """fp32 inputs at head size 128 with a per-dim decay run the whole-sequence
    token-by-token kernel (the state's columns split over four workgroups): a
    ragged length over several 16-token input blocks, mild and strong decays
    (about -20 per token, beyond the chunk kernels' range), the state updated in
    place or written to a new tensor, and groups of up to 16 query heads (two
    head groups per kv head: in place, the reading group runs before the one
    that writes the state)."""
    dtype, D, B, T, Hkv = torch.float32, 128, 2, 97, 2
    Hq = Hkv * G
    seed = 6700 + G + 7 * len(rule) + (0 if mean < 0 else 50)
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=mean)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    state = past.clone()
    dst = state if in_place else torch.empty_like(state)
    if rule == "gated":
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=state, present_state=dst)
        beta = None
    else:
        beta = _beta((B, T, Hkv), dtype, seed)
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=state,
                                           present_state=dst)
    torch.cuda.synchronize()
    assert present.data_ptr() == dst.data_ptr()
    if not in_place:
        assert torch.equal(state, past)
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, rule, past_state=f64(past), decay=f64(g),
                          beta=None if beta is None else f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("kind", ["gated_head", "gated_dim"])
def test_delta_step_strong_decay(dtype, kind):
    """The T = 1 step takes decays of any strength (about -20 here), per head
    or per key dim, for every dtype."""
    B, Hkv, G, D = 2, 2, 4, 64
    Hq = Hkv * G
    q = synth.normal((B, 1, Hq * D), 1.0, dtype, DEV, 7400, "q")
    k = synth.l2_normalized((B, 1, Hkv, D), dtype, DEV, 7400, "k").reshape(B, 1, Hkv * D)
    v = synth.normal((B, 1, Hkv * D), 1.0, dtype, DEV, 7400, "v")
    beta = _beta((B, 1, Hkv), dtype, 7400)
    gshape = (B, 1, Hkv) if kind == "gated_head" else (B, 1, Hkv * D)
    g = synth.logsigmoid_decay(gshape, dtype, DEV, 7400, mean=-20.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 7400, "past")
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated_delta", past_state=f64(past),
                          decay=f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_gated_strong_head_decay(dtype):
    """The per-head gated recurrence with decays of about -20 per token: its
    factors are all exp(later - earlier) <= 1, so no strength overflows."""
    B, T, Hkv, G, D = 2, 300, 2, 2, 64
    Hq = Hkv * G
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, 6600, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, 6600, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, 6600, "v")
    g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, 6600, mean=-20.0)
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(present).all()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", decay=f64(g))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_delta_shared_beta_long(dtype):
    """beta (B,T,1) shared by the kv heads, several chunks, no past state."""
    B, T, Hkv, G, D = 1, 700, 3, 2, 64
    Hq = Hkv * G
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, 81, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, 81, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, 81, "v")
    beta = _beta((B, T, 1), dtype, 81)
    g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, 81, mean=3.0)
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated_delta", decay=f64(g), beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


# ------------------------------------------------------------ gated T=1 step
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("case", ["gated_past_in_place", "gated_no_past", "linear_past"])
def test_gated_step(dtype, D, G, case):
    B, Hkv = 3, 2
    Hq = Hkv * G
    seed = 4000 + D + G
    q = synth.normal((B, 1, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, 1, Hkv, D), dtype, DEV, seed, "k").reshape(B, 1, Hkv * D)
    v = synth.normal((B, 1, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = None if case == "linear_past" else synth.logsigmoid_decay((B, 1, Hkv), dtype, DEV, seed, mean=1.0)
    past = None if case == "gated_no_past" else synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    past_ref = None if past is None else f64(past)
    in_place = case == "gated_past_in_place"
    out, present = la.la_gated_step(q, k, v, Hq, Hkv, decay=g, past_state=past, in_place=in_place)
    torch.cuda.synchronize()
    if in_place:
        assert present.data_ptr() == past.data_ptr()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "linear" if g is None else "gated",
                          past_state=past_ref, decay=None if g is None else f64(g))
    assert out.shape == q.shape
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_gated_prefill_then_steps_equal_full(dtype):
    """A prefill call followed by one-token steps (in place) equals one oracle
    run over the whole sequence, outputs and final state."""
    B, T0, N, Hkv, G, D = 2, 100, 6, 2, 4, 64
    Hq, T = Hkv * G, T0 + N
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, 77, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, 77, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, 77, "v")
    g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, 77, mean=1.0)
    y0, state = la.la_gated_forward(q[:, :T0], k[:, :T0], v[:, :T0], Hq, Hkv, decay=g[:, :T0])
    ys = [y0]
    for t in range(T0, T):
        y, state = la.la_gated_step(q[:, t], k[:, t], v[:, t], Hq, Hkv, decay=g[:, t],
                                    past_state=state, in_place=True)
        ys.append(y[:, None])
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated", decay=f64(g))
    assert_close(torch.cat(ys, 1), oo, TOL[dtype], "outputs")
    assert_close(state, po, TOL[dtype], "state")


GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "onnx_examples.json")))


@pytest.mark.parametrize("ex", [e for e in GOLDEN["examples"] if e["dtype"] == "float32"],
                         ids=lambda e: e["name"])
def test_operator_page_examples_on_gpu(ex):
    """The printed worked examples, zero-padded from head size 2 to 32.

    Padding is exact for every rule: padded q,k dims add 0 to every dot product
    (k^T S and k^T k included), padded v columns give 0 outputs and 0
    pseudo-values, and a per-dim decay gets 0 (no decay) on the padded dims,
    whose rows of S stay 0.  The scale is passed explicitly (the default would
    use the padded head size)."""
    I = ex["inputs"]
    Hq, Hkv = ex["q_num_heads"], ex["kv_num_heads"]
    q, k, v = (np.array(I[n], dtype=np.float32) for n in ("query", "key", "value"))
    B, T = q.shape[:2]
    d = q.shape[-1] // Hq
    P = 32

    def pad(x, H):
        x = x.reshape(B, T, H, d)
        y = np.zeros((B, T, H, P), np.float32)
        y[..., :d] = x
        return torch.from_numpy(y.reshape(B, T, H * P)).to(DEV)

    past = None
    if "past_state" in I:
        p = np.zeros((B, Hkv, P, P), np.float32)
        p[:, :, :d, :d] = np.array(I["past_state"], np.float32)
        past = torch.from_numpy(p).to(DEV)
    decay = None
    if "decay" in I:
        g = np.array(I["decay"], np.float32)
        if g.shape[-1] == Hkv * d and d > 1:  # per key dim
            decay = pad(g, Hkv)
        else:
            decay = torch.from_numpy(g).to(DEV)
    scale = ex.get("scale", 1.0 / np.sqrt(d))
    if ex["update_rule"] in ("delta", "gated_delta"):
        beta = torch.tensor(I["beta"], dtype=torch.float32, device=DEV)
        out, present = la.la_delta_forward(pad(q, Hq), pad(k, Hkv), pad(v, Hkv), Hq, Hkv, beta,
                                           decay=decay, past_state=past, scale=scale)
    else:
        out, present = la.la_gated_forward(pad(q, Hq), pad(k, Hkv), pad(v, Hkv), Hq, Hkv, decay=decay,
                                           past_state=past, scale=scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(B, T, Hq, P)[..., :d].reshape(B, T, Hq * d)
    present = present.cpu().numpy()[:, :, :d, :d]
    np.testing.assert_allclose(out, np.array(ex["output"]), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(present, np.array(ex["present_state"]), rtol=1e-6, atol=1e-6)
