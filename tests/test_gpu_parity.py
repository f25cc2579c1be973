"""Parity of every C-ABI call with the fp64 oracle on seeded inputs (GPU).

Small OPT-shaped workloads (OPT-125m fp32, OPT-6.7B fp16) and ragged shapes whose rows do
not fill a tile; edge cases: empty sets, full sets, t_past = 0, a full cache, B > 1.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (BATCHED_BAR, W_C1, W_C2, W_RAG16, W_RAG32, assert_close, assert_scores_close, chosen_sets, dims_of,
                     kv_host, layer_weights, pred_weights, random_sets, rms, to_dev)

pytestmark = pytest.mark.gpu

WORKLOADS = [W_C1, W_C2, W_RAG16, W_RAG32]
IDS = [w.name for w in WORKLOADS]


@pytest.fixture(scope="module")
def host_layers():
    return {w.name: synth.layer_tensors(w) for w in WORKLOADS}


def batched(w, B):
    return w.with_(batch=B)


# ---------------------------------------------------------------------------
# predictor
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
@pytest.mark.parametrize("B", [1, 3])
def test_predict(dv, host_layers, w, B):
    t = host_layers[w.name]
    x = synth.x_input(batched(w, B), step=5)
    d = to_dev({**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")}, "x": x})
    dims = dims_of(w)
    s_m = torch.empty(B, w.d_ffn, device="cuda")
    s_h = torch.empty(B, w.n_heads, device="cuda")
    ws = dv.workspace(dims, B, w.k, w.kh)
    dv.dv_predict(dims, pred_weights(d), d["x"], s_m, s_h, ws)
    torch.cuda.synchronize()
    rm, rh = oracle.predict(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"], x)
    assert_scores_close(s_m.cpu().numpy(), rm, "s_mlp")
    assert_scores_close(s_h.cpu().numpy(), rh, "s_head")


# ---------------------------------------------------------------------------
# top-k: bit-exact on identical scores
# ---------------------------------------------------------------------------
def score_rows(rng, kind, B, n):
    if kind == "normal":
        return rng.standard_normal((B, n)).astype(np.float32) * 8
    if kind == "ties":
        return (rng.integers(-3, 4, (B, n)) * 0.25).astype(np.float32)
    s = rng.standard_normal((B, n)).astype(np.float32)
    m = rng.random((B, n))
    s[m < 0.05] = -0.0
    s[(m >= 0.05) & (m < 0.08)] = 0.0
    s[(m >= 0.08) & (m < 0.1)] = np.nan
    s[(m >= 0.1) & (m < 0.12)] = np.inf
    s[(m >= 0.12) & (m < 0.14)] = -np.inf
    return s


@pytest.mark.parametrize("n", [1, 7, 12, 96, 1000, 1024, 1025, 3072, 4097, 16384, 36864, 49152, 65536])
@pytest.mark.parametrize("kind", ["normal", "ties", "specials"])
def test_topk_bitexact(dv, n, kind):
    rng = np.random.default_rng(n * 7 + len(kind))
    B = 3
    s = score_rows(rng, kind, B, n)
    sd = torch.from_numpy(s).cuda()
    for k in sorted({0, 1, max(1, n // 20), n // 2, max(0, n - 1), n}):
        out = torch.full((B, max(k, 1)), -7, dtype=torch.int32, device="cuda")
        dv.dv_topk(sd, k, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[:, :k]
        assert np.array_equal(got, oracle.topk(s, k)), (n, kind, k)


# ---------------------------------------------------------------------------
# sparse MLP
# ---------------------------------------------------------------------------
def xn_input(w, B, step=0):
    x = synth.x_input(batched(w, B), step=step)
    return oracle.rmsnorm(x, synth.gains(w)).astype(np.float32)


@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
@pytest.mark.parametrize("case", ["k", "empty", "one", "all", "positive", "batch3"])
def test_sparse_mlp(dv, host_layers, w, case):
    t = host_layers[w.name]
    rng = np.random.default_rng(11)
    B = 3 if case == "batch3" else 1
    xn = xn_input(w, B, step=3)
    F = w.d_ffn
    if case in ("k", "batch3"):
        S = random_sets(rng, B, F, w.k)
    elif case == "empty":
        S = np.zeros((B, 0), np.int32)
    elif case == "one":
        S = np.array([[F - 1]], np.int32)
    elif case == "all":
        S = np.arange(F, dtype=np.int32)[None]
    else:  # exactly the neurons with positive pre-activation: equals the dense MLP
        a = oracle.mlp(xn, t["w1t"], t["b1"], t["w2"], t["b2"], np.ones((1, F)))["a"][0]
        S = np.nonzero(a > 0)[0].astype(np.int32)[None]
    k = S.shape[1]
    d = to_dev({k_: t[k_] for k_ in ("w1t", "b1", "w2", "b2", "wqkv", "bqkv", "wo", "bo", "g1", "g2")})
    dims = dims_of(w)
    xd = torch.from_numpy(xn).cuda()
    Sd = torch.from_numpy(np.ascontiguousarray(S)).cuda() if k > 0 else None
    y = torch.empty(B, w.d_model, device="cuda")
    ws = dv.workspace(dims, B, k, 0)
    dv.dv_sparse_mlp(dims, layer_weights(d), xd, Sd, k, y, ws)
    torch.cuda.synchronize()
    ref = oracle.mlp(xn, t["w1t"], t["b1"], t["w2"], t["b2"], oracle.masks_from_sets(S, F) if k else
                     np.zeros((B, F)))["y_m"]
    got = y.cpu().numpy()
    if case == "empty":
        assert np.array_equal(got, np.broadcast_to(t["b2"], got.shape))
    assert_close(got, ref, w.dtype, f"y_m[{case}]", batch=B)
    if case == "positive":
        dense = oracle.mlp(xn, t["w1t"], t["b1"], t["w2"], t["b2"], np.ones((1, F)))["y_m"]
        assert_close(got, dense, w.dtype, "positive set vs dense")


# ---------------------------------------------------------------------------
# head-sparse attention (+ KV append)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
@pytest.mark.parametrize("case", ["kh", "empty", "all", "t0", "full_cache_batch2"])
def test_sparse_attn(dv, host_layers, w, case):
    t = host_layers[w.name]
    rng = np.random.default_rng(5)
    B = 2 if case == "full_cache_batch2" else 1
    wc = batched(w, B)
    if case == "t0":
        wc = wc.with_(t_past=0)
    H = w.n_heads
    if case == "empty":
        Sh = np.zeros((B, 0), np.int32)
    elif case == "all":
        Sh = np.arange(H, dtype=np.int32)[None]
    else:
        Sh = random_sets(rng, B, H, w.kh)
    kh = Sh.shape[1]
    xn = xn_input(w, B, step=4)
    kc = kv_host(wc, "k_cache")
    vc = kv_host(wc, "v_cache")
    if case == "full_cache_batch2":
        # cache filled to its last slot: t_past = t_max - 1 (the layout's maximum)
        assert wc.t_past == wc.t_max - 1
    dims = dims_of(wc)
    d = to_dev({k_: t[k_] for k_ in ("wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2", "g1", "g2")})
    kcd = torch.from_numpy(kc).cuda()
    vcd = torch.from_numpy(vc).cuda()
    xd = torch.from_numpy(xn).cuda()
    Shd = torch.from_numpy(np.ascontiguousarray(Sh)).cuda() if kh else None
    y = torch.empty(B, w.d_model, device="cuda")
    ws = dv.workspace(dims, B, 0, kh)
    dv.dv_sparse_attn(dims, layer_weights(d), xd, Shd, kh, kcd, vcd, wc.t_past, y, ws)
    torch.cuda.synchronize()
    mask = oracle.masks_from_sets(Sh, H) if kh else np.zeros((B, H))
    ref = oracle.attention(xn, t["wqkv"], t["bqkv"], t["wo"], t["bo"], kc, vc, wc.t_past, mask)
    got = y.cpu().numpy()
    if case == "empty":
        assert np.array_equal(got, np.broadcast_to(t["bo"], got.shape))
    assert_close(got, ref["y_a"], w.dtype, f"y_a[{case}]", batch=B)
    # cache: selected heads gain the current k, v at slot t_past; nothing else changes
    kg, vg = kcd.cpu().numpy(), vcd.cpu().numpy()
    T = wc.t_past
    for b in range(B):
        for h in range(H):
            if h in set(Sh[b].tolist()):
                for m, (got_c, name) in enumerate(((kg, "k"), (vg, "v")), start=1):
                    # the slot holds the fp32 projection rounded to the storage type
                    r = ref["qkv"][b, h, m]
                    ulp = 2.0 ** -10 if w.dtype == "f16" else 2.0 ** -23
                    # batched rows project fp16-rounded inputs on the matrix cores
                    floor = BATCHED_BAR if (w.dtype == "f16" and B >= 2) else 1e-4
                    err = np.abs(got_c[b, h, T].astype(np.float64) - r)
                    assert np.all(err <= ulp * np.abs(r) + floor * rms(r)), f"appended {name}"
                    assert np.max(err) <= 2e-2 * rms(r), f"appended {name}: layer bar"

                    kg_ = got_c[b, h].copy()
                    kg_[T] = (kc if name == "k" else vc)[b, h, T]
                    assert np.array_equal(kg_, (kc if name == "k" else vc)[b, h])
            else:
                assert np.array_equal(kg[b, h], kc[b, h]) and np.array_equal(vg[b, h], vc[b, h])


@pytest.mark.parametrize("w", [W_RAG16, W_RAG32], ids=["ragged-f16", "ragged-f32"])
@pytest.mark.parametrize("raise_late", [False, True], ids=["plain", "later-max"])
def test_sparse_attn_long_cache_several_combine_sweeps(dv, host_layers, w, raise_late):
    """A cache long enough that a head's chunk partials span two sweeps of the combine (over
    5120 keys at 128 keys per block), at batch 2. With raise_late the keys past 5120 are
    scaled up so the largest score sits in the second sweep and the first sweep's sums are
    rescaled to it."""
    t = host_layers[w.name]
    B, T = 2, 6000
    wc = batched(w, B).with_(t_past=T)
    rng = np.random.default_rng(9)
    Sh = random_sets(rng, B, w.n_heads, w.kh)
    kc = kv_host(wc, "k_cache")
    vc = kv_host(wc, "v_cache")
    if raise_late:
        kc = kc.copy()
        kc[:, :, 5200:T] = (kc[:, :, 5200:T].astype(np.float32) * 3).astype(kc.dtype)
    xn = xn_input(w, B, step=6)
    dims = dims_of(wc)
    d = to_dev({k_: t[k_] for k_ in ("wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2", "g1", "g2")})
    y = torch.empty(B, w.d_model, device="cuda")
    dv.dv_sparse_attn(dims, layer_weights(d), torch.from_numpy(xn).cuda(), torch.from_numpy(Sh).cuda(), w.kh,
                      torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), T, y, dv.workspace(dims, B, 0, w.kh))
    torch.cuda.synchronize()
    ref = oracle.attention(xn, t["wqkv"], t["bqkv"], t["wo"], t["bo"], kc, vc, T, oracle.masks_from_sets(Sh, w.n_heads))
    assert_close(y.cpu().numpy(), ref["y_a"], w.dtype, f"y_a[T={T}, later max {raise_late}]", batch=B)


# ---------------------------------------------------------------------------
# layer step
# ---------------------------------------------------------------------------
def run_layer(dv, w, t, x, S=None, Sh=None, inline=False, inplace=False, B=1):
    wc = batched(w, B)
    dims = dims_of(wc)
    d = to_dev({k_: v for k_, v in t.items()})
    kcd = torch.from_numpy(kv_host(wc, "k_cache")).cuda()
    vcd = torch.from_numpy(kv_host(wc, "v_cache")).cuda()
    xd = torch.from_numpy(x).cuda()
    out = xd if inplace else torch.empty_like(xd)
    io = torch.empty(B, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(B, w.kh, dtype=torch.int32, device="cuda")
    ws = dv.workspace(dims, B, w.k, w.kh)
    if inline:
        dv.dv_layer_step(dims, layer_weights(d), pred_weights(d), xd, xd.clone(), w.k, w.kh, None, None, kcd,
                         vcd, wc.t_past, out, io, ho, ws)
    else:
        dv.dv_layer_step(dims, layer_weights(d), None, xd, None, w.k, w.kh,
                         torch.from_numpy(S).cuda(), torch.from_numpy(Sh).cuda(), kcd, vcd, wc.t_past, out,
                         io, ho, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), io.cpu().numpy(), ho.cpu().numpy(), (kcd, vcd)


@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
@pytest.mark.parametrize("B", [1, 2])
def test_layer_step_given_sets(dv, host_layers, w, B):
    t = host_layers[w.name]
    rng = np.random.default_rng(21)
    x = synth.x_input(batched(w, B), step=7)
    S = random_sets(rng, B, w.d_ffn, w.k)
    Sh = random_sets(rng, B, w.n_heads, w.kh)
    got, io, ho, _ = run_layer(dv, w, t, x, S, Sh, B=B)
    assert np.array_equal(io, S) and np.array_equal(ho, Sh)
    wc = batched(w, B)
    ref = oracle.layer(x, t, kv_host(wc, "k_cache"), kv_host(wc, "v_cache"), w.t_past, S, Sh)
    assert_close(got, ref["out"], w.dtype, "layer out", batch=B)
    assert_close(got - ref["h1"], ref["y_m"], w.dtype, "layer y_m", batch=B)


@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
def test_layer_step_inline_prediction(dv, host_layers, w):
    t = host_layers[w.name]
    x = synth.x_input(w, step=9)
    got, io, ho, _ = run_layer(dv, w, t, x, inline=True)
    # inside the library: the sets used are the top-k of its own scores (GPU against GPU)
    dims = dims_of(w)
    d = to_dev({k_: t[k_] for k_ in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")})
    s_m = torch.empty(1, w.d_ffn, device="cuda")
    s_h = torch.empty(1, w.n_heads, device="cuda")
    dv.dv_predict(dims, pred_weights(d), torch.from_numpy(x).cuda(), s_m, s_h, dv.workspace(dims, 1, w.k, w.kh))
    tm = torch.empty(1, w.k, dtype=torch.int32, device="cuda")
    th = torch.empty(1, w.kh, dtype=torch.int32, device="cuda")
    dv.dv_topk(s_m, w.k, tm)
    dv.dv_topk(s_h, w.kh, th)
    torch.cuda.synchronize()
    assert np.array_equal(io, tm.cpu().numpy()) and np.array_equal(ho, th.cpu().numpy())
    # against the oracle's own prediction, selection and layer on the same seeded input
    rm, rh = oracle.predict(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"], x)
    assert_scores_close(s_m.cpu().numpy(), rm, "s_mlp")
    assert_scores_close(s_h.cpu().numpy(), rh, "s_head")
    S = chosen_sets(io, rm, w.k, "neuron set")
    Sh = chosen_sets(ho, rh, w.kh, "head set")
    ref = oracle.layer(x, t, kv_host(w, "k_cache"), kv_host(w, "v_cache"), w.t_past, S, Sh)
    assert_close(got, ref["out"], w.dtype, "layer out (inline sets)")


@pytest.mark.parametrize("w", [W_C2, W_RAG32], ids=["c2", "rag32"])
def test_layer_step_in_place_and_deterministic(dv, host_layers, w):
    t = host_layers[w.name]
    rng = np.random.default_rng(2)
    x = synth.x_input(w, step=1)
    S = random_sets(rng, 1, w.d_ffn, w.k)
    Sh = random_sets(rng, 1, w.n_heads, w.kh)
    a, *_ = run_layer(dv, w, t, x, S, Sh)
    b, *_ = run_layer(dv, w, t, x, S, Sh)
    c, *_ = run_layer(dv, w, t, x, S, Sh, inplace=True)
    assert np.array_equal(a, b), "run-to-run bitwise determinism"
    assert np.array_equal(a, c), "x_out aliasing x gives the same bits"
    assert rms(a) > 0
