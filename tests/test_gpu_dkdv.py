"""Key and value head sizes that differ (the Keras proposal, "Constructor":
value_dim separate from key_dim): q, k (B,T,H,Dk), v and out (B,T,H,Dv), the
state (B,H,Dk,Dv) + (B,H,Dk), each size 32, 64 or 128.  Causal prefill (split
sequences and single passes, masks, initial state), chunked calls chained
with decode steps, and the non-causal path, against the fp64 oracle."""
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
PAIRS = [(64, 128), (128, 64), (32, 128), (128, 32), (32, 64), (64, 32)]
PAIR_IDS = ["%dx%d" % p for p in PAIRS]


def _qkv(B, T, H, Dk, Dv, dtype, seed, qk_std=0.5):
    q = synth.normal((B, T, H, Dk), qk_std, dtype, DEV, seed, "q")
    k = synth.normal((B, T, H, Dk), qk_std, dtype, DEV, seed, "k")
    v = synth.normal((B, T, H, Dv), 1.0, dtype, DEV, seed, "v")
    return q, k, v


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_causal_dk_ne_dv(dtype, dims, fm, norm):
    Dk, Dv = dims
    B, T, H = 2, 200, 3          # split sequences, a ragged tail
    seed = 9600 + Dk + 3 * Dv + 7 * norm
    q, k, v = _qkv(B, T, H, Dk, Dv, dtype, seed)
    mask = synth.random_mask(B, T, 0.85, DEV, seed)
    S0 = synth.normal((B, H, Dk, Dv), 0.5, torch.float32, DEV, seed, "S0")
    Z0 = (synth.normal((B, H, Dk), 1.0, torch.float32, DEV, seed, "Z0").abs() + 0.5) if norm else None
    y, (S, Z) = la.la_forward(q, k, v, mask=mask, state=(S0, Z0), feature_map=fm, use_normalizer=norm,
                              return_state=True)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), mask.cpu().numpy(), f64(S0),
                               f64(Z0) if norm else None, fm, norm, 1e-6)
    tol = TOL[dtype]
    assert y.shape == (B, T, H, Dv) and S.shape == (B, H, Dk, Dv)
    assert_close(y, yo, tol, "out")
    assert_close(S, So, tol, "S")
    if norm:
        assert_close(Z, Zo, tol, "Z")
    assert torch.all(y[~mask.bool()] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("dims", PAIRS, ids=PAIR_IDS)
def test_causal_dk_ne_dv_single_pass(dtype, dims):
    """Enough (batch, head) units for one pass per sequence (no split)."""
    Dk, Dv = dims
    B, T, H = 32, 130, 16
    q, k, v = _qkv(B, T, H, Dk, Dv, dtype, 9700 + Dk + Dv)
    y, (S, Z) = la.la_forward(q, k, v, return_state=True)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    assert_close(y, yo, TOL[dtype], "out")
    assert_close(S, So, TOL[dtype], "S")
    assert_close(Z, Zo, TOL[dtype], "Z")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", PAIRS, ids=PAIR_IDS)
def test_chunked_and_steps_dk_ne_dv(dtype, dims):
    """Chained calls of uneven lengths, then T=1 steps in place, against one
    oracle run over all tokens."""
    Dk, Dv = dims
    B, T, H = 2, 170, 2
    q, k, v = _qkv(B, T, H, Dk, Dv, dtype, 9800 + Dk + Dv)
    state = la.la_initial_state(B, H, Dk, Dv)
    ys = []
    for a, b in ((0, 64), (64, 101), (101, 160)):
        y, state = la.la_forward(q[:, a:b], k[:, a:b], v[:, a:b], state=state, state_out=state,
                                 return_state=True)
        ys.append(y)
    for t in range(160, T):
        y, state = la.la_step(q[:, t], k[:, t], v[:, t], state)
        ys.append(y[:, None])
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v))
    tol = TOL[dtype]
    assert_close(torch.cat(ys, 1), yo, tol, "chunked + steps")
    assert_close(state[0], So, tol, "S")
    assert_close(state[1], Zo, tol, "Z")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
def test_noncausal_dk_ne_dv(dtype, dims, fm):
    Dk, Dv = dims
    B, T, H = 2, 300, 2
    q, k, v = _qkv(B, T, H, Dk, Dv, dtype, 9900 + Dk + Dv, qk_std=1.0)
    mask, _ = synth.right_padding_mask(B, T, DEV, 9900 + Dk, lo=100, hi=T)
    y = la.la_forward(q, k, v, mask=mask, causal=False, feature_map=fm)
    torch.cuda.synchronize()
    yo, _, _ = oracle.noncausal(f64(q), f64(k), f64(v), mask.cpu().numpy(), fm, True, 1e-6)
    assert_close(y, yo, TOL[dtype], "out")
    assert torch.all(y[~mask] == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("dims", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_decode_step_dk_ne_dv(dtype, dims, norm):
    Dk, Dv = dims
    B, H = 3, 5
    q, k, v = _qkv(B, 1, H, Dk, Dv, dtype, 9950 + Dk + Dv)
    S0 = synth.normal((B, H, Dk, Dv), 0.5, torch.float32, DEV, 9950, "S0")
    Z0 = synth.normal((B, H, Dk), 1.0, torch.float32, DEV, 9950, "Z0").abs() + 0.5
    mask = torch.tensor([True, False, True], device=DEV)
    s_kv, s_k = S0.clone(), (Z0.clone() if norm else None)
    y, (S, Z) = la.la_step(q, k, v, (s_kv, s_k), mask=mask, use_normalizer=norm)
    torch.cuda.synchronize()
    yo, So, Zo = oracle.causal(f64(q), f64(k), f64(v), mask.cpu().numpy()[:, None], f64(S0),
                               f64(Z0) if norm else None, "elu_plus_one", norm, 1e-6)
    assert_close(y, yo, TOL[dtype], "out")
    assert_close(S, So, TOL[dtype], "S")
    if norm:
        assert_close(Z, Zo, TOL[dtype], "Z")
    assert torch.all(y[1] == 0) and torch.equal(S[1], S0[1])  # batch row 1 is masked


def test_noalloc_dk_ne_dv():
    """The allocation-free entry point takes unequal head sizes too."""
    B, T, H, Dk, Dv = 4, 1000, 16, 64, 128
    q, k, v = _qkv(B, T, H, Dk, Dv, torch.bfloat16, 9990, 1.0)
    y1 = la.la_forward(q, k, v, causal=False, feature_map="relu")
    y2 = la.la_forward_noalloc(q, k, v, causal=False, feature_map="relu")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
