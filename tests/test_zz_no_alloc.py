"""la_forward_noalloc (the allocation-free la_forward, for callers that cannot
allocate) against la_forward, through the C ABI: two calls in a row on one
stream, the second smaller, each compared element by element with the
workspace entry point's result (same split plan, so the same kernels: equal
bit for bit) and with the fp64 oracle at the floored relative bar."""
import ctypes

import pytest
import torch

import oracle
import synth
import kernelized_linear_attention_chunked_amd as la
from _util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _call(noalloc, q, k, v, mask, causal, fm, state_in=None, with_state=False):
    lib = la.load_library()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[q.dtype]
    out = torch.full((B, T, H, Dv), float("nan"), dtype=q.dtype, device=DEV)
    s_out = (torch.full((B, H, Dk, Dv), float("nan"), device=DEV),
             torch.full((B, H, Dk), float("nan"), device=DEV)) if with_state else (None, None)
    s_in = state_in if state_in is not None else (None, None)
    args = (P(q), P(k), P(v), P(mask), P(s_in[0]), P(s_in[1]), P(s_out[0]), P(s_out[1]), int(causal), fm, 1,
            ctypes.c_float(1e-6), P(out), B, T, H, Dk, Dv, code)
    if noalloc:
        rc = lib.la_forward_noalloc(*args, _stream())
    else:
        n = ctypes.c_size_t(0)
        assert lib.la_workspace_size(B, T, H, Dk, Dv, code, int(causal), ctypes.byref(n)) == 0
        ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=DEV)
        rc = lib.la_forward(*args, P(ws), n.value, _stream())
    assert rc == 0, lib.la_last_error_message().decode()
    return out, s_out


def test_noalloc_matches_forward_two_calls():
    # call 1: non-causal, masked, 1000 (batch, head) units at head size 128:
    # one split per unit, 66 MB of the 64 MiB scratch
    B, T, H, D = 8, 200, 125, 128
    q, k, v = synth.qkv(B, T, H, D, torch.bfloat16, DEV, 71, 1.0, 1.0, 1.0)
    mask, _ = synth.right_padding_mask(B, T, DEV, 71)
    m8 = mask.to(torch.uint8).contiguous()
    print("call 1: non-causal", (B, T, H, D), flush=True)
    y_na, _ = _call(True, q, k, v, m8, False, 1)
    y_ws, _ = _call(False, q, k, v, m8, False, 1)
    # call 2 (smaller): causal split sequence with a state in and out, fp32
    B2, T2, H2, D2 = 1, 1000, 2, 64
    q2, k2, v2 = synth.qkv(B2, T2, H2, D2, torch.float32, DEV, 72)
    S0 = torch.randn((B2, H2, D2, D2), device=DEV) * 0.3
    Z0 = torch.rand((B2, H2, D2), device=DEV) + 0.5
    print("call 2: causal split", (B2, T2, H2, D2), flush=True)
    y2_na, st_na = _call(True, q2, k2, v2, None, True, 0, (S0, Z0), True)
    y2_ws, st_ws = _call(False, q2, k2, v2, None, True, 0, (S0, Z0), True)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws)
    assert torch.equal(y2_na, y2_ws)
    assert torch.equal(st_na[0], st_ws[0]) and torch.equal(st_na[1], st_ws[1])
    yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), mask.cpu().numpy(), "relu", True, 1e-6)
    assert_close(y_na, yo, TOL[torch.bfloat16], "call 1 out")
    yo2, So2, Zo2 = oracle.causal(f64(q2), f64(k2), f64(v2), None, f64(S0), f64(Z0))
    assert_close(y2_na, yo2, TOL[torch.float32], "call 2 out")
    assert_close(st_na[0], So2, TOL[torch.float32], "call 2 S")
    assert_close(st_na[1], Zo2, TOL[torch.float32], "call 2 Z")


def test_noalloc_split_workloads_repeated():
    """The split plans of the D=64 causal and D=128 non-causal workload shapes
    (smaller T), twice each in a row: the scratch keeps the previous call's
    contents, which no call may depend on."""
    cases = [((8, 512, 16, 64), True, 0), ((4, 2048, 16, 128), False, 1)]
    for rep in range(2):
        for (B, T, H, D), causal, fm in cases:
            q, k, v = synth.qkv(B, T, H, D, torch.bfloat16, DEV, 73 + rep, 0.5, 0.5, 1.0)
            mask = None if causal else synth.right_padding_mask(B, T, DEV, 73 + rep)[0].to(torch.uint8)
            print("rep", rep, "causal" if causal else "non-causal", (B, T, H, D), flush=True)
            y_na, s_na = _call(True, q, k, v, mask, causal, fm, None, causal)
            y_ws, s_ws = _call(False, q, k, v, mask, causal, fm, None, causal)
            torch.cuda.synchronize()
            assert torch.equal(y_na, y_ws)
            if causal:
                assert torch.equal(s_na[0], s_ws[0]) and torch.equal(s_na[1], s_ws[1])
