"""The delta rules split over T (the LinearAttention operator page, "Description":
update rules "delta" and "gated_delta", any chunk-parallel evaluation with the
sequential result).  With few (batch, kv head) units the library runs each
segment's state map S_end = M S_start + N from S = I with zero values and from
S = 0, composes the start states, and runs every segment with outputs.  The
split results match the fp64 oracle and the unsplit evaluation (no workspace)
for both rules, every decay kind, every dtype, ragged segments, a past state,
strong per-dim decays (the token-by-token fallback inside a segment), and a
config-5-shaped gated-delta call (B=2, Hkv=8, Hq=32, T=32768, 16 segments)."""
import ctypes

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


def _inputs(B, T, Hq, Hkv, D, dtype, seed, kind, mean=1.0):
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = None
    if kind == "head":
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=mean)
    elif kind == "dim":
        g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=mean)
    beta = torch.sigmoid(synth.normal((B, T, Hkv), 1.0, torch.float32, DEV, seed, "beta")).to(dtype)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    return q, k, v, g, beta, past


def _workspace_bytes(B, T, Hq, Hkv, D, dtype, per_dim):
    n = ctypes.c_size_t(0)
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype]
    lib = la.load_library()
    assert lib.la_delta_workspace_size(B, T, Hq, Hkv, D, D, code, int(per_dim), ctypes.byref(n)) == 0
    return n.value


def _unsplit(q, k, v, g, beta, past, Hq, Hkv, D, per_dim):
    """la_delta_forward through the C ABI without a workspace (no split)."""
    B, T, _ = q.shape
    lib = la.load_library()
    out = torch.empty_like(q)
    pres = torch.empty((B, Hkv, D, D), dtype=torch.float32, device=DEV)
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[q.dtype]
    p = lambda t: ctypes.c_void_p(0 if t is None else t.data_ptr())
    rc = lib.la_delta_forward(p(q), p(k), p(v), p(g), int(per_dim), p(beta), 1, p(past), p(pres), p(out), B, T,
                              Hq, Hkv, D, D, code, ctypes.c_float(0.0), None, 0,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    return out, pres


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("kind", ["none", "head", "dim"])
@pytest.mark.parametrize("G", [1, 4])
def test_delta_split_matches_oracle_and_unsplit(dtype, kind, G):
    # 2 units, 16 chunks: 4 segments of 256 tokens, the last one ragged (232)
    B, T, Hkv = 1, 1000, 2
    D = 64 if (dtype == torch.float32 and kind == "dim") else 128
    Hq = Hkv * G
    seed = 7700 + G + 10 * ["none", "head", "dim"].index(kind)
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, dtype, seed, kind)
    assert _workspace_bytes(B, T, Hq, Hkv, D, dtype, kind == "dim") == D * D * 4 * (2 * 3 * 2 + 2 * 4 + 1)
    out, pres = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    out_u, pres_u = _unsplit(q, k, v, g, beta, past, Hq, Hkv, D, kind == "dim")
    torch.cuda.synchronize()
    rule = "delta" if kind == "none" else "gated_delta"
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, rule, past_state=f64(past),
                          decay=None if g is None else f64(g), beta=f64(beta))
    tol = TOL[dtype]
    e1 = assert_close(out, oo, tol, "out (split)")
    e2 = assert_close(pres, po, tol, "present_state (split)")
    e3 = assert_close(out_u, oo, tol, "out (unsplit)")
    e4 = assert_close(pres_u, po, tol, "present_state (unsplit)")
    print("split out %.2e state %.2e | unsplit out %.2e state %.2e" % (e1, e2, e3, e4), flush=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_delta_split_strong_perdim_decay(dtype):
    """Per-dim decays of about -4 per token: segments re-evaluate token by token,
    including the map passes (from S = I, zero values)."""
    B, T, Hkv, G, D = 1, 700, 2, 2, 64
    Hq = Hkv * G
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, dtype, 7800, "dim", mean=-4.0)
    assert _workspace_bytes(B, T, Hq, Hkv, D, dtype, True) > 0
    out, pres = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated_delta", past_state=f64(past), decay=f64(g),
                          beta=f64(beta))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(pres, po, TOL[dtype], "present_state")


def test_delta_split_in_place_state():
    """present_state == past_state with a split: the start states are composed
    from the past state before the last segment overwrites it."""
    B, T, Hkv, G, D = 1, 900, 1, 2, 128
    Hq = Hkv * G
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, torch.bfloat16, 7850, "head")
    ref_past = past.clone()
    out, pres = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past, present_state=past)
    torch.cuda.synchronize()
    assert pres.data_ptr() == past.data_ptr()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, "gated_delta", past_state=f64(ref_past), decay=f64(g),
                          beta=f64(beta))
    assert_close(out, oo, TOL[torch.bfloat16], "out")
    assert_close(pres, po, TOL[torch.bfloat16], "present_state")


def test_delta_split_config5_shape():
    """B=2, Hkv=8, Hq=32, T=32768, head size 128, bf16, gated delta with a
    per-head decay: 16 units in 16 segments (256 workgroups per pass).  Units
    (batch 0, kv head 0), (batch 1, kv head 5) and (batch 1, kv head 7) against
    the oracle over all 32768 tokens, every output of the call finite."""
    B, T, Hq, Hkv, D, G = 2, 32768, 32, 8, 128, 4
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, torch.bfloat16, 7900, "head")
    E = D * D * 4
    assert _workspace_bytes(B, T, Hq, Hkv, D, torch.bfloat16, False) == E * (16 * 15 * 2 + 16 * 16 + 1)
    out, pres = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(pres).all()
    for b, j in ((0, 0), (1, 5), (1, 7)):
        qs = q[b:b + 1, :, j * G * D:(j + 1) * G * D]
        ks, vs = k[b:b + 1, :, j * D:(j + 1) * D], v[b:b + 1, :, j * D:(j + 1) * D]
        gs, bs = g[b:b + 1, :, j:j + 1], beta[b:b + 1, :, j:j + 1]
        oo, po = oracle.la_op(f64(qs), f64(ks), f64(vs), G, 1, "gated_delta", past_state=f64(past[b:b + 1, j:j + 1]),
                              decay=f64(gs), beta=f64(bs))
        e1 = assert_close(out[b:b + 1, :, j * G * D:(j + 1) * G * D], oo, 2e-2, "out unit (%d, %d)" % (b, j))
        e2 = assert_close(pres[b:b + 1, j:j + 1], po, 2e-2, "present_state unit (%d, %d)" % (b, j))
        print("unit (%d, %d): out %.2e state %.2e" % (b, j, e1, e2), flush=True)
