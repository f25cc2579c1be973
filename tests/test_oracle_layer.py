"""Pins for the oracle's norm, sparse MLP, head-sparse attention and layer (CPU only).

Sources: DejaVu Guide, "The Contextual Sparsity Hypothesis" (ReLU makes inactive
neurons exact zeros), "The Synchronous Prediction Dilemma" (FFN equation),
"Head-Pruned Attention Dispatch", "Step-by-Step Implementation" (layer sketch).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


# --------------------------------------------------------------------------
# brute-force references written as plain loops (tiny shapes only)
# --------------------------------------------------------------------------

def loops_rmsnorm(x, g, eps=1e-5):
    ms = sum(v * v for v in x) / len(x)
    return [g[i] * x[i] / math.sqrt(ms + eps) for i in range(len(x))]


def loops_mlp(x, w1t, b1, w2, b2, S):
    d, F = len(x), len(w1t)
    y = list(b2)
    for j in range(F):
        if j not in S:
            continue
        a = b1[j] + sum(x[c] * w1t[j][c] for c in range(d))
        u = a if a > 0 else 0.0
        for c in range(d):
            y[c] += u * w2[j][c]
    return y


def loops_attention(xn, wqkv, bqkv, wo, bo, kc, vc, T, heads):
    H, _, dh, d = len(wqkv), 3, len(wqkv[0][0]), len(xn)
    y = list(bo)
    for h in range(H):
        if h not in heads:
            continue
        proj = [[bqkv[h][m][e] + sum(xn[c] * wqkv[h][m][e][c] for c in range(d)) for e in range(dh)]
                for m in range(3)]
        q, kk, vv = proj
        keys = [kc[h][t] for t in range(T)] + [kk]
        vals = [vc[h][t] for t in range(T)] + [vv]
        sc = [sum(q[e] * key[e] for e in range(dh)) / math.sqrt(dh) for key in keys]
        mx = max(sc)
        ex = [math.exp(s - mx) for s in sc]
        tot = sum(ex)
        o = [sum(ex[t] / tot * vals[t][e] for t in range(len(keys))) for e in range(dh)]
        for c in range(len(bo)):
            y[c] += sum(o[e] * wo[h][e][c] for e in range(dh))
    return y


def tiny_layer(rng, d=8, F=10, H=2, dh=4, T=3, bias=True):
    s = 0.5
    t = {
        "g1": rng.uniform(0.5, 1.5, d), "g2": rng.uniform(0.5, 1.5, d),
        "wqkv": rng.standard_normal((H, 3, dh, d)) * s,
        "bqkv": rng.standard_normal((H, 3, dh)) * s * bias,
        "wo": rng.standard_normal((H, dh, d)) * s, "bo": rng.standard_normal(d) * s * bias,
        "w1t": rng.standard_normal((F, d)) * s, "b1": rng.standard_normal(F) * s * bias,
        "w2": rng.standard_normal((F, d)) * s, "b2": rng.standard_normal(d) * s * bias,
    }
    kc = rng.standard_normal((1, H, T + 1, dh))
    vc = rng.standard_normal((1, H, T + 1, dh))
    x = rng.standard_normal((1, d))
    return t, kc, vc, x


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def test_rmsnorm_constant_rows_closed_form():
    for c in (-3.0, 0.25, 7.0):
        x = np.full((1, 16), c)
        g = np.linspace(0.5, 2.0, 16)
        np.testing.assert_allclose(oracle.rmsnorm(x, g)[0], g * c / math.sqrt(c * c + 1e-5),
                                   rtol=1e-14)


def test_rmsnorm_loops_and_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 33))
    g = rng.uniform(0.5, 1.5, 33)
    got = oracle.rmsnorm(x, g)
    for b in range(3):
        np.testing.assert_allclose(got[b], loops_rmsnorm(x[b].tolist(), g.tolist()), rtol=1e-12)
    # scaling x by c and eps by c^2 leaves the result unchanged
    np.testing.assert_allclose(oracle.rmsnorm(x * 1e4, g, eps=1e-5 * 1e8), got, rtol=1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean((got / g) ** 2, axis=-1)), 1.0, rtol=1e-5)


# --------------------------------------------------------------------------
# MLP
# --------------------------------------------------------------------------

def mlp_case(seed, d=12, F=9, B=1, bias=True):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, d)), rng.standard_normal((F, d)),
            rng.standard_normal(F) * bias, rng.standard_normal((F, d)), rng.standard_normal(d) * bias)


def test_mlp_all_subsets_brute_force():
    x, w1t, b1, w2, b2 = mlp_case(0, d=5, F=7)
    for k in range(8):
        for S in itertools.combinations(range(7), k):
            got = oracle.mlp(x, w1t, b1, w2, b2, oracle.masks_from_sets([list(S)], 7))["y_m"][0]
            ref = loops_mlp(x[0].tolist(), w1t.tolist(), b1.tolist(), w2.tolist(), b2.tolist(), set(S))
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mlp_all_selected_is_torch_dense():
    x, w1t, b1, w2, b2 = mlp_case(1, d=64, F=256, B=3)
    ref = torch.nn.functional.linear(
        torch.relu(torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w1t),
                                              torch.from_numpy(b1))),
        torch.from_numpy(w2.T.copy()), torch.from_numpy(b2)).numpy()
    got = oracle.mlp(x, w1t, b1, w2, b2, np.ones((3, 256)))["y_m"]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mlp_positive_set_and_supersets_reproduce_dense():
    x, w1t, b1, w2, b2 = mlp_case(2, d=64, F=256)
    dense = oracle.mlp(x, w1t, b1, w2, b2, np.ones((1, 256)))
    pos = np.nonzero(dense["a"][0] > 0)[0]
    got = oracle.mlp(x, w1t, b1, w2, b2, oracle.masks_from_sets([pos], 256))["y_m"]
    assert np.max(np.abs(got - dense["y_m"])) <= 1e-12
    rng = np.random.default_rng(0)
    extra = rng.choice(np.setdiff1d(np.arange(256), pos), 20, replace=False)
    sup = np.sort(np.concatenate([pos, extra]))
    got2 = oracle.mlp(x, w1t, b1, w2, b2, oracle.masks_from_sets([sup], 256))["y_m"]
    assert np.max(np.abs(got2 - dense["y_m"])) <= 1e-12
    # dropping one positive neuron changes the output
    drop = oracle.mlp(x, w1t, b1, w2, b2, oracle.masks_from_sets([pos[1:]], 256))["y_m"]
    assert np.max(np.abs(drop - dense["y_m"])) > 1e-6


def test_mlp_empty_set_gives_b2_and_homogeneity():
    x, w1t, b1, w2, b2 = mlp_case(3)
    np.testing.assert_array_equal(oracle.mlp(x, w1t, b1, w2, b2, np.zeros((1, 9)))["y_m"][0], b2)
    x, w1t, b1, w2, b2 = mlp_case(4, bias=False)
    m = oracle.masks_from_sets([[0, 2, 3, 7]], 9)
    np.testing.assert_allclose(oracle.mlp(2 * x, w1t, b1, w2, b2, m)["y_m"],
                               2 * oracle.mlp(x, w1t, b1, w2, b2, m)["y_m"], rtol=1e-13, atol=1e-13)


def test_mlp_compacted_rows_equal_masked_dense():
    """Passing only the selected rows with an all-ones mask equals the masked dense form.

    Large-shape parity checks rely on this identity to avoid materialising
    every row of the weights on the host.
    """
    x, w1t, b1, w2, b2 = mlp_case(5, d=48, F=300, B=2)
    S = np.sort(np.random.default_rng(0).choice(300, 37, replace=False))
    full = oracle.mlp(x, w1t, b1, w2, b2, oracle.masks_from_sets([S, S], 300))["y_m"]
    comp = oracle.mlp(x, w1t[S], b1[S], w2[S], b2, np.ones((2, 37)))["y_m"]
    np.testing.assert_allclose(comp, full, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attn_case(seed, d=16, H=4, dh=4, T=5, B=1):
    rng = np.random.default_rng(seed)
    return dict(xn=rng.standard_normal((B, d)), wqkv=rng.standard_normal((H, 3, dh, d)) * 0.4,
                bqkv=rng.standard_normal((H, 3, dh)) * 0.4, wo=rng.standard_normal((H, dh, d)),
                bo=rng.standard_normal(d), k_cache=rng.standard_normal((B, H, T + 1, dh)),
                v_cache=rng.standard_normal((B, H, T + 1, dh)), t_past=T)


@pytest.mark.parametrize("heads", [[0], [1, 3], [0, 1, 2, 3], []])
def test_attention_brute_force(heads):
    c = attn_case(0)
    got = oracle.attention(head_mask=oracle.masks_from_sets([heads], 4), **c)["y_a"][0]
    ref = loops_attention(c["xn"][0].tolist(), c["wqkv"].tolist(), c["bqkv"].tolist(), c["wo"].tolist(),
                          c["bo"].tolist(), c["k_cache"][0].tolist(), c["v_cache"][0].tolist(),
                          c["t_past"], set(heads))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_attention_t0_returns_v():
    c = attn_case(1, T=0)
    out = oracle.attention(head_mask=np.ones((1, 4)), **c)
    qkv = out["qkv"][0]
    np.testing.assert_allclose(out["o"][0], qkv[:, 2], rtol=1e-14)


def test_attention_equal_keys_give_mean_of_values():
    c = attn_case(2, T=6)
    # zero key weights and biases: every key (cached and current) equals the cached row 0 = 0
    c["wqkv"][:, 1] = 0.0
    c["bqkv"][:, 1] = 0.0
    c["k_cache"][:] = 0.0
    out = oracle.attention(head_mask=np.ones((1, 4)), **c)
    v_cur = out["qkv"][0, :, 2]
    mean = (c["v_cache"][0, :, :6].sum(axis=1) + v_cur) / 7.0
    np.testing.assert_allclose(out["o"][0], mean, rtol=1e-13)


def test_attention_per_head_additivity_and_empty():
    c = attn_case(3, H=5)
    sel = [0, 2, 4]
    full = oracle.attention(head_mask=oracle.masks_from_sets([sel], 5), **c)["y_a"][0]
    parts = sum(oracle.attention(head_mask=oracle.masks_from_sets([[h]], 5), **c)["y_a"][0] - c["bo"]
                for h in sel)
    np.testing.assert_allclose(full - c["bo"], parts, rtol=1e-12, atol=1e-12)
    empty = oracle.attention(head_mask=np.zeros((1, 5)), **c)["y_a"][0]
    np.testing.assert_array_equal(empty, c["bo"])


def test_attention_dense_matches_torch_sdpa():
    c = attn_case(4, d=32, H=4, dh=8, T=9)
    out = oracle.attention(head_mask=np.ones((1, 4)), **c)
    qkv = out["qkv"][0]
    q = torch.from_numpy(qkv[:, 0][:, None, :])                          # [H][1][dh]
    K = torch.from_numpy(np.concatenate([c["k_cache"][0, :, :9], qkv[:, 1][:, None]], axis=1))
    V = torch.from_numpy(np.concatenate([c["v_cache"][0, :, :9], qkv[:, 2][:, None]], axis=1))
    o = torch.nn.functional.scaled_dot_product_attention(q, K, V).numpy()[:, 0]
    np.testing.assert_allclose(out["o"][0], o, rtol=1e-12, atol=1e-12)


def test_attention_compacted_heads_equal_masked_dense():
    c = attn_case(5, H=6)
    sel = np.array([1, 4])
    full = oracle.attention(head_mask=oracle.masks_from_sets([sel], 6), **c)["y_a"]
    cc = dict(c)
    for name in ("wqkv", "bqkv", "wo"):
        cc[name] = c[name][sel]
    cc["k_cache"] = c["k_cache"][:, sel]
    cc["v_cache"] = c["v_cache"][:, sel]
    comp = oracle.attention(head_mask=np.ones((1, 2)), **cc)["y_a"]
    np.testing.assert_allclose(comp, full, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# layer
# --------------------------------------------------------------------------

def loops_layer(x, t, kc, vc, T, S, Sh):
    xn1 = loops_rmsnorm(x, t["g1"])
    ya = loops_attention(xn1, t["wqkv"], t["bqkv"], t["wo"], t["bo"], kc, vc, T, Sh)
    h1 = [x[i] + ya[i] for i in range(len(x))]
    xn2 = loops_rmsnorm(h1, t["g2"])
    ym = loops_mlp(xn2, t["w1t"], t["b1"], t["w2"], t["b2"], S)
    return [h1[i] + ym[i] for i in range(len(x))]


@pytest.mark.parametrize("seed", range(4))
def test_layer_brute_force(seed):
    rng = np.random.default_rng(seed)
    t, kc, vc, x = tiny_layer(rng)
    S = sorted(rng.choice(10, 4, replace=False).tolist())
    Sh = [int(rng.integers(0, 2))]
    got = oracle.layer(x, t, kc, vc, 3, [S], [Sh])["out"][0]
    tl = {k: v.tolist() for k, v in t.items()}
    ref = loops_layer(x[0].tolist(), tl, kc[0].tolist(), vc[0].tolist(), 3, set(S), set(Sh))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_planted_dropped_bias_is_caught(monkeypatch):
    """Dropping b1 inside the oracle's MLP must fail the brute-force pin."""
    real = oracle.dejavu.mlp

    def wrong(xn, w1t, b1, w2, b2, mask):
        return real(xn, w1t, np.zeros_like(np.asarray(b1, np.float64)), w2, b2, mask)
    monkeypatch.setattr(oracle.dejavu, "mlp", wrong)
    with pytest.raises(AssertionError):
        test_layer_brute_force(0)


def test_planted_wrong_attention_scale_is_caught(monkeypatch):
    """Leaving out the 1/sqrt(dh) scale must fail the brute-force pin."""
    class NoSqrt:
        sqrt = staticmethod(lambda v: 1.0)
    monkeypatch.setattr(oracle.dejavu, "math", NoSqrt)
    with pytest.raises(AssertionError):
        test_attention_brute_force([1, 3])
