"""GQA group sizes beyond 8 query heads per kv head, and group sizes that are
not powers of two (the LinearAttention operator page, "Description": q_num_heads
is any positive multiple of kv_num_heads; multi-query is kv_num_heads = 1).
The chunk kernels run such a group as several workgroups of 8, 4, 2 or 1 query
heads, each with the kv head's recurrence; the one-token steps read the heads
out in passes.  Every rule, prefill (split sequences included) and T = 1,
against the fp64 oracle."""
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
RULES = ["linear", "gated", "gated_perdim", "delta", "gated_delta"]


def _inputs(B, T, Hq, Hkv, D, dtype, seed, rule):
    q = synth.normal((B, T, Hq * D), 1.0, dtype, DEV, seed, "q")
    k = synth.l2_normalized((B, T, Hkv, D), dtype, DEV, seed, "k").reshape(B, T, Hkv * D)
    v = synth.normal((B, T, Hkv * D), 1.0, dtype, DEV, seed, "v")
    g = None
    if rule in ("gated", "gated_delta"):
        g = synth.logsigmoid_decay((B, T, Hkv), dtype, DEV, seed, mean=1.0)
    elif rule == "gated_perdim":
        g = synth.logsigmoid_decay((B, T, Hkv * D), dtype, DEV, seed, mean=1.0)
    beta = None
    if rule.endswith("delta"):
        beta = torch.sigmoid(synth.normal((B, T, Hkv), 1.0, torch.float32, DEV, seed, "beta")).to(dtype)
    past = synth.normal((B, Hkv, D, D), 0.3, torch.float32, DEV, seed, "past")
    return q, k, v, g, beta, past


def _run(q, k, v, g, beta, past, Hq, Hkv, rule):
    if rule.endswith("delta"):
        return la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past)
    return la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past)


def _oracle(q, k, v, g, beta, past, Hq, Hkv, rule):
    r = "gated" if rule == "gated_perdim" else rule
    return oracle.la_op(f64(q), f64(k), f64(v), Hq, Hkv, r, past_state=f64(past),
                        decay=None if g is None else f64(g), beta=None if beta is None else f64(beta))


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("G", [3, 6, 12, 16, 32])
@pytest.mark.parametrize("rule", RULES)
def test_group_sizes_prefill(dtype, G, rule):
    B, T, Hkv, D = 1, 190, 2, 64      # 2 units: split sequences for the gated rules
    Hq = Hkv * G
    seed = 8100 + G + 11 * RULES.index(rule)
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, dtype, seed, rule)
    out, present = _run(q, k, v, g, beta, past, Hq, Hkv, rule)
    torch.cuda.synchronize()
    oo, po = _oracle(q, k, v, g, beta, past, Hq, Hkv, rule)
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("G", [3, 12, 16, 32])
@pytest.mark.parametrize("rule", RULES)
def test_group_sizes_step(dtype, G, rule):
    """T = 1 (the state-streaming step kernels), in place."""
    B, Hkv, D = 3, 2, 128
    Hq = Hkv * G
    seed = 8200 + G + 11 * RULES.index(rule)
    q, k, v, g, beta, past = _inputs(B, 1, Hq, Hkv, D, dtype, seed, rule)
    ref_past = past.clone()
    if rule.endswith("delta"):
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past, present_state=past)
    else:
        out, present = la.la_gated_step(q, k, v, Hq, Hkv, decay=g, past_state=past, in_place=True)
    torch.cuda.synchronize()
    oo, po = _oracle(q, k, v, g, beta, ref_past, Hq, Hkv, rule)
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("rule", ["gated", "gated_perdim", "gated_delta"])
def test_multi_query_32_to_1(dtype, rule):
    """Hq = 32 query heads on one kv head at head size 128, a sequence long
    enough to split (4 query-head groups per segment)."""
    B, T, Hq, Hkv, D = 2, 1100, 32, 1, 128
    seed = 8300 + RULES.index(rule)
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, dtype, seed, rule)
    out, present = _run(q, k, v, g, beta, past, Hq, Hkv, rule)
    torch.cuda.synchronize()
    oo, po = _oracle(q, k, v, g, beta, past, Hq, Hkv, rule)
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("G", [16, 32])
@pytest.mark.parametrize("rule", RULES)
def test_group_sizes_single_pass_in_place(dtype, G, rule):
    """One pass per sequence (a single ragged chunk: no split) with the state
    updated in place by several query-head groups, each of which reads the
    past state at its start: the groups that only read it run before group 0,
    which writes it.  288 units, so the workgroups do not all fit the GPU at
    once."""
    B, T, Hkv, D = 144, 60, 2, 64
    Hq = Hkv * G
    seed = 8400 + G + 11 * RULES.index(rule)
    q, k, v, g, beta, past = _inputs(B, T, Hq, Hkv, D, dtype, seed, rule)
    ref_past = past.clone()
    if rule.endswith("delta"):
        out, present = la.la_delta_forward(q, k, v, Hq, Hkv, beta, decay=g, past_state=past, present_state=past)
    else:
        out, present = la.la_gated_forward(q, k, v, Hq, Hkv, decay=g, past_state=past, present_state=past)
    torch.cuda.synchronize()
    assert present.data_ptr() == past.data_ptr()
    oo, po = _oracle(q, k, v, g, beta, ref_past, Hq, Hkv, rule)
    assert_close(out, oo, TOL[dtype], "out")
    assert_close(present, po, TOL[dtype], "present_state")
