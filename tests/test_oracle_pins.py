"""Pins for the fp64 oracle (CPU only).

The oracle is the plain per-token recurrence.  These tests tie it to things other
than itself:

* the worked examples printed on the LinearAttention operator page (values in
  tests/golden/onnx_examples.json, each with its citation);
* the seeded causal-vs-non-causal mean absolute difference printed on the
  "Causal Linear Attention" page (Brenndoerfer), In[22]/Out[23];
* brute-force quadratic forms phi(Q) phi(K)^T on tiny inputs, written here
  independently of the recurrence (the only place a T x T matrix appears);
* closed forms for special inputs and invariants the Keras proposal's test plan
  names (chunked == full, token-by-token == full, masks, GQA == replicated MHA).

A planted mistake anywhere in the recurrence (dropped diagonal, wrong eps
placement, transposed S, wrong decay axis, wrong GQA grouping, mask by
multiplication) fails at least one of them.
"""
import json
import os
import zlib

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EXAMPLES = json.load(open(os.path.join(GOLDEN, "onnx_examples.json")))["examples"]


def _phi(x, fm, eps):
    if fm == "elu_plus_one":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    return np.maximum(x, 0.0) + eps


# ---------------------------------------------------------------- printed values
@pytest.mark.parametrize("ex", [e for e in EXAMPLES if e["dtype"] == "float32"],
                         ids=lambda e: e["name"])
def test_operator_page_examples_fp32(ex):
    I = ex["inputs"]
    out, present = oracle.la_op(I["query"], I["key"], I["value"], ex["q_num_heads"],
                                ex["kv_num_heads"], ex["update_rule"],
                                past_state=I.get("past_state"), decay=I.get("decay"),
                                beta=I.get("beta"), scale=ex.get("scale", 0.0))
    # printed to ~8 significant digits of an fp32 computation
    np.testing.assert_allclose(out, np.array(ex["output"]), rtol=2e-7, atol=2e-7)
    np.testing.assert_allclose(present, np.array(ex["present_state"]), rtol=2e-7, atol=2e-7)


def test_operator_page_example_fp16():
    ex = [e for e in EXAMPLES if e["dtype"] == "float16"][0]
    I = {k: np.array(v, dtype=np.float16).astype(np.float64) for k, v in ex["inputs"].items()}
    out, present = oracle.la_op(I["query"], I["key"], I["value"], ex["q_num_heads"],
                                ex["kv_num_heads"], ex["update_rule"], decay=I["decay"],
                                beta=I["beta"])
    # printed with 4 significant digits after an fp16 round of the result
    for got, want in ((out, ex["output"]), (present, ex["present_state"])):
        got16 = got.astype(np.float16).astype(np.float64)
        want = np.array(want)
        assert np.all(np.abs(got16 - want) <= 1e-3 * np.maximum(np.abs(want), 1.0))


def _p2_inputs():
    # The page's own recipe: legacy MT19937 seed 42, randn(32,16)*0.5 for Q then K,
    # randn for V, all float32.
    rs = np.random.RandomState(42)
    n, d = 32, 16
    Q = rs.randn(n, d).astype(np.float32) * 0.5
    K = rs.randn(n, d).astype(np.float32) * 0.5
    V = rs.randn(n, d).astype(np.float32)
    return Q[None, :, None], K[None, :, None], V[None, :, None]


def test_brenndoerfer_seeded_difference():
    q, k, v = _p2_inputs()
    yc, _, _ = oracle.causal(q, k, v, eps=1e-6)
    yn, _, _ = oracle.noncausal(q, k, v, eps=1e-6)
    diff = np.mean(np.abs(yc - yn))
    assert round(diff, 4) == 0.2188, diff


def test_brenndoerfer_figure_rejects_excluded_diagonal():
    # Shows the pin discriminates: a readout that excludes the current token
    # (y_t from S_{t-1}) gives a different 4-digit figure.  Shifting q by one
    # token turns the oracle's inclusive readout into the exclusive one.
    q, k, v = _p2_inputs()
    qs = np.concatenate([q[:, 1:], q[:, :1]], axis=1)
    y_incl_shift, _, _ = oracle.causal(qs, k, v)
    y_excl = np.concatenate([np.zeros_like(y_incl_shift[:, :1]), y_incl_shift[:, :-1]], axis=1)
    yn, _, _ = oracle.noncausal(q, k, v)
    assert round(np.mean(np.abs(y_excl - yn)), 4) != 0.2188


# ------------------------------------------------------------ brute-force forms
def _brute_causal(q, k, v, mask, S0, Z0, fm, norm, eps):
    """y = (phiQ S0 + A V) / (phiQ Z0 + A 1 + eps), A = phiQ phiK^T * tril * m m^T."""
    B, T, H, Dk = q.shape
    y = np.zeros(v.shape)
    for b in range(B):
        m = np.ones(T, bool) if mask is None else mask[b].astype(bool)
        for h in range(H):
            fq = _phi(q[b, :, h], fm, eps)
            fk = _phi(k[b, :, h], fm, eps)
            A = (fq @ fk.T) * np.tril(np.ones((T, T))) * m[None, :]
            vv = np.where(m[:, None], v[b, :, h], 0.0)
            s0 = np.zeros((Dk, v.shape[-1])) if S0 is None else S0[b, h]
            z0 = np.zeros(Dk) if Z0 is None else Z0[b, h]
            num = fq @ s0 + A @ vv
            den = fq @ z0 + A.sum(1) + eps
            yy = num / den[:, None] if norm else num
            y[b, :, h] = np.where(m[:, None], yy, 0.0)
    return y


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("mask_kind", ["none", "right", "left", "gaps"])
def test_causal_matches_bruteforce(fm, norm, with_state, mask_kind):
    rng = np.random.default_rng(zlib.crc32(repr((fm, norm, with_state, mask_kind)).encode()))
    B, T, H, Dk, Dv = 2, 23, 3, 5, 4
    q, k = _rand(rng, B, T, H, Dk, scale=0.7), _rand(rng, B, T, H, Dk, scale=0.7)
    v = _rand(rng, B, T, H, Dv)
    mask = {"none": None,
            "right": np.arange(T)[None, :] < np.array([[T], [15]]),
            "left": np.arange(T)[None, :] >= np.array([[3], [0]]),
            "gaps": rng.random((B, T)) > 0.3}[mask_kind]
    S0 = np.abs(_rand(rng, B, H, Dk, Dv)) if with_state else None
    Z0 = np.abs(_rand(rng, B, H, Dk)) + 1 if with_state else None
    y, S, Z = oracle.causal(q, k, v, mask, S0, Z0, fm, norm, 1e-6)
    yb = _brute_causal(q, k, v, mask, S0, Z0, fm, norm, 1e-6)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)
    # final state = initial + sum over valid tokens (independent of token order)
    m = np.ones((B, T), bool) if mask is None else mask.astype(bool)
    fk = _phi(k, fm, 1e-6) * m[:, :, None, None]
    S_ref = np.einsum("bthd,bthe->bhde", fk, v * m[:, :, None, None])
    Z_ref = fk.sum(1)
    if with_state:
        S_ref, Z_ref = S_ref + S0, Z_ref + Z0
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Z, Z_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
@pytest.mark.parametrize("norm", [True, False])
def test_noncausal_matches_bruteforce(fm, norm):
    rng = np.random.default_rng(7 + norm + 2 * (fm == "relu"))
    B, T, H, D = 2, 19, 2, 6
    q, k, v = _rand(rng, B, T, H, D), _rand(rng, B, T, H, D), _rand(rng, B, T, H, D)
    mask = np.arange(T)[None, :] < np.array([[T], [11]])
    y, _, _ = oracle.noncausal(q, k, v, mask, fm, norm, 1e-6)
    for b in range(B):
        m = mask[b]
        for h in range(H):
            fq, fk = _phi(q[b, :, h], fm, 1e-6), _phi(k[b, :, h], fm, 1e-6)
            A = (fq @ fk.T) * m[None, :]            # (T,T): queries x keys, invalid keys out
            num = A @ v[b, :, h]                     # (phiQ phiK^T) V, the other association
            den = A.sum(1) + 1e-6
            want = num / den[:, None] if norm else num
            want[~m] = 0.0
            np.testing.assert_allclose(y[b, :, h], want, rtol=1e-12, atol=1e-12)


def _brute_gated(q, k, v, g, past, G, scale, per_dim):
    """o_i = scale [ q_i^T (D_{0..i} S0) + sum_{j<=i} (q_i * D_{j+1..i}) . k_j  v_j ]."""
    B, T, Hq, Dk = q.shape
    Hkv, Dv = k.shape[2], v.shape[-1]
    out = np.zeros((B, T, Hq, Dv))
    for b in range(B):
        for h in range(Hq):
            j = h // G
            gg = g[b, :, j] if per_dim else np.repeat(g[b, :, j:j + 1], Dk, axis=1)  # (T,Dk)
            cs = np.concatenate([np.zeros((1, Dk)), np.cumsum(gg, 0)])            # cs[t] = sum_{s<t}
            for i in range(T):
                acc = (q[b, i, h] * np.exp(cs[i + 1])) @ past[b, j]
                for jj in range(i + 1):
                    w = np.exp(cs[i + 1] - cs[jj + 1])
                    acc = acc + ((q[b, i, h] * w) @ k[b, jj, j]) * v[b, jj, j]
                out[b, i, h] = scale * acc
    return out


@pytest.mark.parametrize("per_dim", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_gated_matches_bruteforce(per_dim, G):
    rng = np.random.default_rng(100 + G + 10 * per_dim)
    B, T, Hkv, Dk, Dv = 2, 13, 2, 3, 4
    Hq = Hkv * G
    q, k, v = _rand(rng, B, T, Hq, Dk), _rand(rng, B, T, Hkv, Dk), _rand(rng, B, T, Hkv, Dv)
    g = -np.abs(_rand(rng, B, T, Hkv, Dk if per_dim else 1, scale=0.3))
    g = g if per_dim else g[..., 0]
    past = _rand(rng, B, Hkv, Dk, Dv)
    scale = 0.37
    out, present = oracle.la_op(q.reshape(B, T, -1), k.reshape(B, T, -1), v.reshape(B, T, -1), Hq,
                                Hkv, "gated", past_state=past, decay=g.reshape(B, T, -1),
                                scale=scale)
    want = _brute_gated(q, k, v, g, past, G, scale, per_dim)
    np.testing.assert_allclose(out.reshape(want.shape), want, rtol=1e-11, atol=1e-11)
    # present state: decayed past plus decayed sum of outer products
    gg = g if per_dim else np.repeat(g[..., None], Dk, axis=-1)
    tot = gg.sum(1)                                          # (B,Hkv,Dk)
    suf = tot[:, None] - np.cumsum(gg, 1)                    # sum_{s>j}
    S_ref = np.exp(tot)[..., None] * past + np.einsum("bjhd,bjhe->bhde", k * np.exp(suf), v)
    np.testing.assert_allclose(present, S_ref, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ closed forms
def test_causal_closed_form_constant_features():
    # q = k = 0 with elu+1 gives phi == 1: y_t = (t*Dk)/(t*Dk + eps) * mean(v_1..v_t)
    rng = np.random.default_rng(3)
    B, T, H, D = 1, 17, 2, 8
    z = np.zeros((B, T, H, D))
    v = _rand(rng, B, T, H, D)
    eps = 1e-3
    y, S, Z = oracle.causal(z, z, v, eps=eps)
    t = np.arange(1, T + 1)[None, :, None, None]
    want = (t * D) / (t * D + eps) * np.cumsum(v, 1) / t
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Z, np.full((B, H, D), float(T)), rtol=0, atol=0)
    yn, _, _ = oracle.noncausal(z, z, v, eps=eps)
    np.testing.assert_allclose(yn, np.broadcast_to(T * D / (T * D + eps) * v.mean(1, keepdims=True),
                                                    yn.shape), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
def test_single_token_closed_form(fm):
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 1, 1, 6), _rand(rng, 1, 1, 1, 6), _rand(rng, 1, 1, 1, 5)
    eps = 1e-2
    a = _phi(q, fm, eps)[0, 0, 0] @ _phi(k, fm, eps)[0, 0, 0]
    y, _, _ = oracle.causal(q, k, v, feature_map=fm, eps=eps)
    np.testing.assert_allclose(y[0, 0, 0], a / (a + eps) * v[0, 0, 0], rtol=1e-14)
    y, _, _ = oracle.causal(q, k, v, feature_map=fm, use_normalizer=False, eps=eps)
    np.testing.assert_allclose(y[0, 0, 0], a * v[0, 0, 0], rtol=1e-14)


def test_gated_full_forgetting_and_zero_decay():
    rng = np.random.default_rng(5)
    B, T, H, D = 1, 6, 2, 3
    q, k, v = _rand(rng, B, T, H * D), _rand(rng, B, T, H * D), _rand(rng, B, T, H * D)
    # g = 0 reduces "gated" to "linear"
    o1, s1 = oracle.la_op(q, k, v, H, H, "gated", decay=np.zeros((B, T, H)))
    o2, s2 = oracle.la_op(q, k, v, H, H, "linear")
    np.testing.assert_allclose(o1, o2, rtol=0, atol=0)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=0)
    # exp(g) = 0 forgets everything: o_t = scale (q_t . k_t) v_t
    o3, s3 = oracle.la_op(q, k, v, H, H, "gated", decay=np.full((B, T, H), -1e4), scale=0.5)
    qq, kk, vv = (x.reshape(B, T, H, D) for x in (q, k, v))
    want = 0.5 * np.einsum("bthd,bthd->bth", qq, kk)[..., None] * vv
    np.testing.assert_allclose(o3.reshape(want.shape), want, rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------------- invariants
def test_chunked_and_token_by_token_equal_full():
    rng = np.random.default_rng(6)
    B, T, H, D = 2, 37, 2, 5
    q, k, v = _rand(rng, B, T, H, D, scale=.5), _rand(rng, B, T, H, D, scale=.5), _rand(rng, B, T, H, D)
    mask = rng.random((B, T)) > 0.2
    y, S, Z = oracle.causal(q, k, v, mask)
    ys, S1, Z1 = [], None, None
    for a, b in ((0, 10), (10, 11), (11, 30), (30, 37)):
        yc, S1, Z1 = oracle.causal(q[:, a:b], k[:, a:b], v[:, a:b], mask[:, a:b], S1, Z1)
        ys.append(yc)
    np.testing.assert_allclose(np.concatenate(ys, 1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S, rtol=1e-13)
    np.testing.assert_allclose(Z1, Z, rtol=1e-13)
    S1 = Z1 = None
    for t in range(T):
        yt, S1, Z1 = oracle.causal(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], mask[:, t:t + 1], S1, Z1)
        np.testing.assert_allclose(yt[:, 0], y[:, t], rtol=1e-13, atol=1e-13)


def test_masked_positions_are_selected_out():
    rng = np.random.default_rng(8)
    B, T, H, D = 1, 20, 1, 4
    q, k, v = _rand(rng, B, T, H, D), _rand(rng, B, T, H, D), _rand(rng, B, T, H, D)
    mask = np.ones((B, T), bool)
    mask[0, [3, 4, 11, 19]] = False
    y, S, Z = oracle.causal(q, k, v, mask, feature_map="relu")
    # NaN garbage at masked positions reaches nothing
    qn, kn, vn = q.copy(), k.copy(), v.copy()
    for a in (qn, kn, vn):
        a[0, ~mask[0]] = np.nan
    y2, S2, Z2 = oracle.causal(qn, kn, vn, mask, feature_map="relu")
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(S2, S)
    assert np.all(y[0, ~mask[0]] == 0.0)
    # removing the masked tokens gives the same valid outputs and state
    keep = mask[0]
    y3, S3, Z3 = oracle.causal(q[:, keep], k[:, keep], v[:, keep], feature_map="relu")
    np.testing.assert_allclose(y3, y[:, keep], rtol=1e-13)
    np.testing.assert_allclose(S3, S, rtol=1e-13)
    # all-false mask: zero output, state passes through
    S0, Z0 = np.abs(_rand(rng, B, H, D, D)), np.abs(_rand(rng, B, H, D))
    y4, S4, Z4 = oracle.causal(q, k, v, np.zeros((B, T), bool), S0, Z0)
    assert np.all(y4 == 0.0)
    np.testing.assert_array_equal(S4, S0)
    np.testing.assert_array_equal(Z4, Z0)
    # all-true mask is no mask
    y5, _, _ = oracle.causal(q, k, v, np.ones((B, T), bool))
    y6, _, _ = oracle.causal(q, k, v)
    np.testing.assert_array_equal(y5, y6)


def test_noncausal_permutation_invariance():
    rng = np.random.default_rng(9)
    B, T, H, D = 1, 15, 2, 4
    q, k, v = _rand(rng, B, T, H, D), _rand(rng, B, T, H, D), _rand(rng, B, T, H, D)
    y, S, Z = oracle.noncausal(q, k, v, feature_map="relu")
    p = rng.permutation(T)
    y2, S2, Z2 = oracle.noncausal(q, k[:, p], v[:, p], feature_map="relu")
    np.testing.assert_allclose(y2, y, rtol=1e-12)


def test_gqa_equals_replicated_mha():
    rng = np.random.default_rng(10)
    B, T, Hkv, G, D = 2, 9, 2, 3, 4
    Hq = Hkv * G
    q, k, v = _rand(rng, B, T, Hq * D), _rand(rng, B, T, Hkv * D), _rand(rng, B, T, Hkv * D)
    g = -np.abs(_rand(rng, B, T, Hkv, scale=0.2))
    out, present = oracle.la_op(q, k, v, Hq, Hkv, "gated", decay=g)
    rep = lambda x: np.repeat(x.reshape(B, T, Hkv, -1), G, axis=2).reshape(B, T, -1)
    out2, present2 = oracle.la_op(q, rep(k), rep(v), Hq, Hq, "gated", decay=np.repeat(g, G, axis=2))
    np.testing.assert_allclose(out2, out, rtol=1e-13)
    np.testing.assert_allclose(present2[:, ::G], present, rtol=1e-13)


# ------------------------------------------------------------- gradients (backward)
@pytest.mark.parametrize("fm", ["elu_plus_one", "relu"])
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
def test_backward_matches_finite_differences(fm, norm):
    """The oracle backward against central differences of the fp64 forward, for
    the loss sum(dy*y) + sum(dS*S_T) + sum(dZ*Z_T), every input element, with a
    mask (invalid tokens get zero gradients) and an initial state (Keras
    proposal, "Stability": float64 numerical-gradient checks)."""
    rng = np.random.default_rng(11 + 2 * norm + (fm == "relu"))
    B, T, H, Dk, Dv = 2, 7, 2, 3, 2
    q = rng.normal(size=(B, T, H, Dk))
    k = rng.normal(size=(B, T, H, Dk))
    v = rng.normal(size=(B, T, H, Dv))
    S0 = rng.normal(size=(B, H, Dk, Dv)) * 0.5
    Z0 = rng.uniform(0.5, 2.0, size=(B, H, Dk))
    mask = np.ones((B, T), bool)
    mask[0, 2] = mask[1, 5] = mask[1, 0] = False
    dy = rng.normal(size=(B, T, H, Dv))
    dS = rng.normal(size=(B, H, Dk, Dv))
    dZ = rng.normal(size=(B, H, Dk)) if norm else None
    # keep inputs off relu's kink
    for x in (q, k):
        x[np.abs(x) < 1e-3] = 0.5

    def loss(q_, k_, v_, S0_, Z0_):
        y, S, Z = oracle.causal(q_, k_, v_, mask, S0_, Z0_ if norm else None, fm, norm, 1e-6)
        out = np.sum(dy * y) + np.sum(dS * S)
        if norm:
            out += np.sum(dZ * Z)
        return out

    args = [q, k, v, S0, Z0]
    dq, dk, dv, dS0, dZ0 = oracle.causal_backward(q, k, v, dy, mask, S0, Z0 if norm else None, dS, dZ,
                                                  fm, norm, 1e-6)
    grads = [dq, dk, dv, dS0, dZ0]
    h = 1e-6
    for a in range(4 if not norm else 5):
        fd = np.zeros_like(args[a])
        for idx in np.ndindex(args[a].shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[a][idx] += h
            minus[a][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(grads[a], fd, rtol=1e-5, atol=1e-6, err_msg="argument %d" % a)
    # invalid tokens: no gradient to q, k, v
    for b, t in ((0, 2), (1, 5), (1, 0)):
        assert not np.any(dq[b, t]) and not np.any(dk[b, t]) and not np.any(dv[b, t])
