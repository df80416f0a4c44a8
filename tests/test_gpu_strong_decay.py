"""Decays of any strength (the LinearAttention operator page, "Description",
puts no bound on the log-space decay).  The chunk kernels factorise the
in-chunk decay relative to a reference token; where a cumulative decay inside
a chunk passes the factors' safe range, the workgroup re-evaluates its tokens
one at a time.  These tests drive both regimes: per-key-dim decays of about -4
and -20 per token (RWKV-6-like strengths), one strong dimension in one chunk
of an otherwise weakly decaying sequence, and fp16 delta inputs with strong
per-head decays; gated and gated-delta rules, split sequences and single
passes, against the fp64 oracle."""
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


def _inputs(B, T, Hq, Hkv, D, dtype, seed, mean, per_dim=True):
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = synth.logsigmoid_decay((B, T, Hkv * D) if per_dim else (B, T, Hkv), dtype, DEV, seed, mean=mean)
    beta = torch.sigmoid(synth.normal((B, T, Hkv), 1.0, torch.float32, DEV, seed, "beta")).to(dtype)
    return q, k, v, g, beta


def _check(out, present, q, k, v, g, beta, Hq, Hkv, rule, dtype, past=None):
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(present).all()
    oo, po = oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, rule, decay=f64(g),
                          beta=None if beta is None else f64(beta),
                          past_state=None if past is None else f64(past))
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("mean", [-4.0, -20.0], ids=["m4", "m20"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_gated_perdim_very_strong(dtype, mean, D, G):
    # 2 units of 5 chunks: split sequences
    B, T, Hkv = 1, 300, 2
    Hq = Hkv * G
    q, k, v, g, _ = _inputs(B, T, Hq, Hkv, D, dtype, 9100 + D + G, mean)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 9100 + D, "past")
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)
    _check(out, present, q, k, v, g, None, Hq, Hkv, "gated", dtype, past)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_gated_perdim_very_strong_single_pass(dtype):
    """Enough units for one pass per sequence (no split), decays about -4."""
    B, T, Hkv, G, D = 64, 200, 8, 2, 64
    Hq = Hkv * G
    q, k, v, g, _ = _inputs(B, T, Hq, Hkv, D, dtype, 9200, -4.0)
    out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g)
    _check(out, present, q, k, v, g, None, Hq, Hkv, "gated", dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("rule", ["gated", "gated_delta"])
def test_one_strong_dimension_in_one_chunk(dtype, rule):
    """Weak decays everywhere except dimension 5 of kv head 1 in tokens
    130..160, where each token decays by 8 (-240 in all): only the chunks
    around it leave the factorised range."""
    B, T, Hkv, G, D = 1, 330, 2, 2, 64
    Hq = Hkv * G
    q, k, v, g, beta = _inputs(B, T, Hq, Hkv, D, dtype, 9300, 2.0)
    g = g.float()
    g[0, 130:160, 1 * D + 5] = -8.0
    g = g.to(dtype)
    if rule == "gated":
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g)
        beta = None
    else:
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g)
    _check(out, present, q, k, v, g, beta, Hq, Hkv, rule, dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("mean", [-4.0, -20.0], ids=["m4", "m20"])
@pytest.mark.parametrize("per_dim", [True, False], ids=["perdim", "perhead"])
def test_gated_delta_very_strong(dtype, mean, per_dim):
    B, T, Hkv, G, D = 1, 260, 2, 4, 64
    Hq = Hkv * G
    q, k, v, g, beta = _inputs(B, T, Hq, Hkv, D, dtype, 9400 + int(-mean), mean, per_dim)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 9400, "past")
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    _check(out, present, q, k, v, g, beta, Hq, Hkv, "gated_delta", dtype, past)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_gated_delta_very_strong_d128(dtype):
    B, T, Hkv, G, D = 2, 200, 1, 8, 128
    Hq = Hkv * G
    q, k, v, g, beta = _inputs(B, T, Hq, Hkv, D, dtype, 9500, -4.0)
    out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g)
    _check(out, present, q, k, v, g, beta, Hq, Hkv, "gated_delta", dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("rule", ["gated", "gated_delta"])
def test_strong_perdim_single_pass_in_place(dtype, rule):
    """One pass per sequence (no split, no workspace), a past state updated in
    place, decays of about -4 per token: the token-by-token re-evaluation
    starts from the past state, not from a state the pass has already written."""
    B, T, Hkv, G, D = 64, 200, 8, 2, 64
    Hq = Hkv * G
    q, k, v, g, beta = _inputs(B, T, Hq, Hkv, D, dtype, 9600, -4.0)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 9600, "past")
    state = past.clone()
    if rule == "gated":
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=state, present_state=state)
        beta = None
    else:
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=state, present_state=state)
    assert present.data_ptr() == state.data_ptr()
    _check(out, present, q, k, v, g, beta, Hq, Hkv, rule, dtype, past)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("G", [2, 16])
@pytest.mark.parametrize("layout", ["single_pass_in_place", "split"])
def test_strong_perdim_some_segments_groups(dtype, G, layout):
    """Strong per-dim decays in some (unit, segment) pairs only, with one or
    several query-head groups per kv head: the flagged pairs are re-evaluated
    token by token for every group (outputs, and the final state from group
    0), the others keep the chunk pass's results.  The single pass updates the
    state in place (288 units of one chunk); the split call has 2 units of 6
    segments."""
    Hkv, D = 2, 64
    B, T = (144, 60) if layout == "single_pass_in_place" else (1, 330)
    Hq = Hkv * G
    q, k, v, g, _ = _inputs(B, T, Hq, Hkv, D, dtype, 9700 + G, 2.0)
    g = g.float()
    # about -180 and -80 accumulated inside a chunk: past the factorised range
    if layout == "single_pass_in_place":
        g[0::3, 10:40, 3] = -6.0
        g[1::3, 20:30, D + 7] = -8.0
    else:
        g[0, 70:100, 3] = -6.0
        g[0, 260:270, D + 7] = -8.0
    g = g.to(dtype)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, 9700 + G, "past")
    if layout == "single_pass_in_place":
        state = past.clone()
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=state, present_state=state)
        assert present.data_ptr() == state.data_ptr()
    else:
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)
    _check(out, present, q, k, v, g, None, Hq, Hkv, "gated", dtype, past)
