"""The chunk-parallel causal backward (16-bit inputs, head sizes 32 and 64):
gradients of the normalized causal recurrence ("[Feature] LinearAttention layer
for Keras", "Stability" and "Acceptance": recurrent/parallel gradient parity
and float64 checks) against the fp64 oracle backward.  Unequal key and value
head sizes ("Constructor": value_dim), one pass per sequence and split
sequences, sequence lengths around the 32-token chunk and 64-token segment
grid, initial state and final-state gradient, masks with whole masked chunks
and NaN in the masked tokens."""
import pytest
import torch

import oracle
import synth
import kernelized_linear_attention_chunked_amd as la
from _util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DTYPES = [torch.bfloat16, torch.float16]
DT_IDS = ["bf16", "f16"]


def _inputs(B, T, H, Dk, Dv, dtype, seed):
    q = synth.normal((B, T, H, Dk), 0.5, dtype, DEV, seed, "q")
    k = synth.normal((B, T, H, Dk), 0.5, dtype, DEV, seed, "k")
    v = synth.normal((B, T, H, Dv), 1.0, dtype, DEV, seed, "v")
    dy = synth.normal((B, T, H, Dv), 1.0, dtype, DEV, seed, "dy")
    return q, k, v, dy


def _states(B, H, Dk, Dv, seed):
    S0 = synth.normal((B, H, Dk, Dv), 0.5, torch.float32, DEV, seed, "S0")
    Z0 = synth.normal((B, H, Dk), 1.0, torch.float32, DEV, seed, "Z0").abs() + 0.5
    gS = synth.normal((B, H, Dk, Dv), 0.2, torch.float32, DEV, seed, "gS")
    gZ = synth.normal((B, H, Dk), 0.2, torch.float32, DEV, seed, "gZ")
    return S0, Z0, gS, gZ


def _check(got, q, k, v, dy, mask=None, state=None, dstate=None, fm="elu_plus_one", norm=True, tol=2e-2):
    torch.cuda.synchronize()
    dq, dk, dv, (dS0, dZ0) = got
    m = None if mask is None else mask.cpu().numpy() != 0
    S0, Z0 = state if state is not None else (None, None)
    gS, gZ = dstate if dstate is not None else (None, None)
    ref = oracle.causal_backward(f64(q), f64(k), f64(v), f64(dy), m, None if S0 is None else f64(S0),
                                 None if (Z0 is None or not norm) else f64(Z0), None if gS is None else f64(gS),
                                 None if (gZ is None or not norm) else f64(gZ), feature_map=fm,
                                 use_normalizer=norm)
    errs = {}
    for x, y, what in ((dq, ref[0], "dq"), (dk, ref[1], "dk"), (dv, ref[2], "dv"), (dS0, ref[3], "dS0")):
        errs[what] = assert_close(x, y, tol, what)
    if norm:
        errs["dZ0"] = assert_close(dZ0, ref[4], tol, "dZ0")
    print(" ".join("%s %.2e" % kv for kv in errs.items()), flush=True)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", [(32, 64), (64, 32), (32, 32), (64, 64)], ids=["32x64", "64x32", "32", "64"])
@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_backward_head_sizes(dtype, dims, fm, norm):
    """Split sequences (6 units), a ragged tail, a mask, state and dstate."""
    Dk, Dv = dims
    B, T, H = 2, 200, 3
    seed = 9100 + Dk + 3 * Dv + 7 * norm + 11 * (fm == "relu")
    q, k, v, dy = _inputs(B, T, H, Dk, Dv, dtype, seed)
    S0, Z0, gS, gZ = _states(B, H, Dk, Dv, seed)
    mask = synth.random_mask(B, T, 0.85, DEV, seed)
    st = (S0, Z0 if norm else None)
    ds = (gS, gZ if norm else None)
    got = la.la_backward(q, k, v, dy, mask=mask, state=st, dstate=ds, feature_map=fm, use_normalizer=norm)
    assert got[0].shape == q.shape and got[2].shape == v.shape and got[3][0].shape == (B, H, Dk, Dv)
    _check(got, q, k, v, dy, mask, st, ds, fm, norm, TOL[dtype])
    invalid = ~mask.bool()
    for g in got[:3]:
        assert not g[invalid].float().abs().sum()


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", [(64, 64), (32, 64)], ids=["64", "32x64"])
def test_backward_one_pass_per_sequence(dtype, dims):
    """512 units: every sequence in one segment (no split, no slots)."""
    Dk, Dv = dims
    B, T, H = 32, 100, 16
    q, k, v, dy = _inputs(B, T, H, Dk, Dv, dtype, 9200 + Dk + Dv)
    S0, Z0, gS, gZ = _states(B, H, Dk, Dv, 9200)
    got = la.la_backward(q, k, v, dy, state=(S0, Z0), dstate=(gS, gZ))
    _check(got, q, k, v, dy, None, (S0, Z0), (gS, gZ), tol=TOL[dtype])


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 63, 64, 65, 127, 129, 500])
def test_backward_lengths(T):
    """Lengths around the 32-token chunk and the 64-token segment grid."""
    B, H, D = 1, 2, 64
    q, k, v, dy = _inputs(B, T, H, D, D, torch.bfloat16, 9300 + T)
    S0, Z0, gS, gZ = _states(B, H, D, D, 9300 + T)
    got = la.la_backward(q, k, v, dy, state=(S0, Z0), dstate=(gS, gZ))
    _check(got, q, k, v, dy, None, (S0, Z0), (gS, gZ))


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
def test_backward_masked_chunks_with_nan(dtype):
    """Whole masked 32- and 64-token blocks, a masked head and tail, and NaN in
    every masked token's q, k, v and dy: the gradients stay finite, exactly 0
    at masked tokens, and match the oracle on the valid ones."""
    B, T, H, D = 2, 300, 2, 64
    q, k, v, dy = _inputs(B, T, H, D, D, dtype, 9400)
    mask = torch.ones((B, T), dtype=torch.bool, device=DEV)
    mask[0, 32:64] = False
    mask[0, 128:192] = False
    mask[1, :40] = False
    mask[1, 250:] = False
    ref_in = [t.clone() for t in (q, k, v, dy)]
    for t in (q, k, v, dy):
        t[~mask] = float("nan")
    got = la.la_backward(q, k, v, dy, mask=mask)
    for g in got[:3]:
        assert torch.isfinite(g.float()).all()
        assert not g[~mask].float().abs().sum()
    for t in ref_in:
        t[~mask] = 0
    _check(got, *ref_in, mask, tol=TOL[dtype])


def test_backward_every_head_size_pair():
    """A short sequence (two segments, a ragged chunk) at every head-size pair."""
    for Dk in (32, 64):
        for Dv in (32, 64):
            q, k, v, dy = _inputs(1, 70, 1, Dk, Dv, torch.bfloat16, 9500 + Dk + Dv)
            got = la.la_backward(q, k, v, dy)
            _check(got, q, k, v, dy)


@pytest.mark.parametrize("T", [64, 128, 320, 512, 576, 1536], ids=lambda t: "T%d" % t)
def test_backward_segment_counts(T):
    """One unit: 1, 2, 5, 8, 9 and 24 segments of 64 tokens.  Up to 8 the
    passes add the unprefixed segment sums themselves; beyond, a prefix pass
    runs over them.  Initial state and final-state gradient included."""
    B, H, D = 1, 1, 64
    q, k, v, dy = _inputs(B, T, H, D, D, torch.bfloat16, 9600 + T)
    S0, Z0, gS, gZ = _states(B, H, D, D, 9600 + T)
    got = la.la_backward(q, k, v, dy, state=(S0, Z0), dstate=(gS, gZ))
    _check(got, q, k, v, dy, None, (S0, Z0), (gS, gZ))
