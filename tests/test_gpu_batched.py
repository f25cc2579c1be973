"""Batched decode against the fp64 oracle applied row by row (GPU). Batches of 3..32 rows
with fp16 weights run on the union of the rows' selections (matrix cores); 2 rows run row
by row; both are covered.

Each row's result depends only on its own neuron and head sets; the union only shares the
weight reads. Rows draw their sets from a Zipf(1.1)-skewed popularity (Gumbel-top-k of
log-popularity, the batched workload's selection rule), so the rows overlap the way the
batched workload's do. The batched path rounds the activations (normalised inputs, ReLU
outputs, attention outputs, predictor stage-1 outputs) to fp16 for the matrix cores; its
internal bar BATCHED_BAR allows for that rounding (about 2^-11 relative per operand),
and the layer bar 2e-2 * RMS(ref) applies unchanged. The predictor's activations are
split into fp16 high parts and remainders, so its scores meet the single-row bar.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (BATCHED_BAR, LAYER_TOL, W_C2, W_RAG16, assert_scores_close, chosen_sets, dims_of, kv_host,
                     layer_weights, pred_weights, random_sets, rms, to_dev)

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def host_layers():
    return {w.name: synth.layer_tensors(w) for w in (W_C2, W_RAG16)}


def close(got, ref, what, bar=BATCHED_BAR):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = max(rms(ref), 1e-30)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= LAYER_TOL * scale, f"{what}: max-abs {err:.3e} > {LAYER_TOL} * RMS {scale:.3e}"
    assert err <= bar * scale, f"{what}: max-abs {err:.3e} > batched bar {bar} * RMS {scale:.3e}"
    return err / scale


def zipf_sets(w, B, n, k, name):
    sc = synth.zipf_scores(w.with_(batch=B), n, name)
    return np.asarray(oracle.topk(sc, k), np.int32).reshape(B, k)


def run_layer(dv, w, t, x, S, Sh, ws=None):
    B = x.shape[0]
    dims = dims_of(w)
    d = to_dev(t)
    wc = w.with_(batch=B)
    kcd = torch.from_numpy(kv_host(wc, "k_cache")).cuda()
    vcd = torch.from_numpy(kv_host(wc, "v_cache")).cuda()
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    k, kh = S.shape[1], Sh.shape[1]
    ws = dv.workspace(dims, B, k, kh) if ws is None else ws
    # an empty set still passes a valid (unread) index buffer
    Sd = torch.from_numpy(S).cuda() if k > 0 else torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    Shd = torch.from_numpy(Sh).cuda() if kh > 0 else torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    dv.dv_layer_step(dims, layer_weights(d), None, xd, None, k, kh, Sd, Shd, kcd, vcd, w.t_past, out, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kcd.cpu().numpy(), vcd.cpu().numpy()


@pytest.mark.parametrize("w", [W_C2, W_RAG16], ids=["opt6.7b-shape", "ragged"])
@pytest.mark.parametrize("B", [2, 3, 5, 8, 16, 17, 32])
def test_batched_layer_matches_rowwise_oracle(dv, host_layers, w, B):
    t = host_layers[w.name]
    wc = w.with_(batch=B)
    x = synth.x_input(wc, step=11)
    S = zipf_sets(w, B, w.d_ffn, w.k, "sel_mlp")
    Sh = zipf_sets(w, B, w.n_heads, w.kh, "sel_head")
    got, kc, vc = run_layer(dv, w, t, x, S, Sh)
    ref = oracle.layer(x, t, kv_host(wc, "k_cache"), kv_host(wc, "v_cache"), w.t_past, S, Sh)
    close(got, ref["out"], f"B={B} layer out")
    close(got - ref["h1"], ref["y_m"], f"B={B} y_m")
    # the current token's k/v land in slot t_past of every (row, selected head) only
    qkv = ref["qkv"]   # [B][H][3][dh] fp64
    for b in range(B):
        for h in range(w.n_heads):
            kslot, vslot = kc[b, h, w.t_past].astype(np.float64), vc[b, h, w.t_past].astype(np.float64)
            if h in Sh[b]:
                kk, vv = qkv[b, h, 1], qkv[b, h, 2]
                assert np.max(np.abs(kslot - kk)) <= BATCHED_BAR * 4 * max(rms(kk), 1e-30) + 2 ** -10 * np.max(np.abs(kk))
                assert np.max(np.abs(vslot - vv)) <= BATCHED_BAR * 4 * max(rms(vv), 1e-30) + 2 ** -10 * np.max(np.abs(vv))
            else:
                assert not kslot.any() and not vslot.any(), f"row {b} head {h} not selected but slot written"


def test_batched_rows_equal_single_rows(dv, host_layers):
    """Each row of a batched step agrees with that row run alone (B = 1 path, fp32
    activations) within the batched bar: the union never changes a row's selection."""
    w = W_RAG16
    t = host_layers[w.name]
    B = 9
    x = synth.x_input(w.with_(batch=B), step=3)
    S = zipf_sets(w, B, w.d_ffn, w.k, "sel_mlp")
    Sh = zipf_sets(w, B, w.n_heads, w.kh, "sel_head")
    got, *_ = run_layer(dv, w, t, x, S, Sh)
    for b in range(B):
        # a single-row step on the same row's cache (row b of the batched caches)
        wc = w.with_(batch=B)
        kcb = kv_host(wc, "k_cache")[b:b + 1].copy()
        vcb = kv_host(wc, "v_cache")[b:b + 1].copy()
        dims = dims_of(w)
        d = to_dev(t)
        xd = torch.from_numpy(x[b:b + 1].copy()).cuda()
        out = torch.empty_like(xd)
        dv.dv_layer_step(dims, layer_weights(d), None, xd, None, w.k, w.kh, torch.from_numpy(S[b:b + 1].copy()).cuda(),
                         torch.from_numpy(Sh[b:b + 1].copy()).cuda(), torch.from_numpy(kcb).cuda(),
                         torch.from_numpy(vcb).cuda(), w.t_past, out, ws=dv.workspace(dims, 1, w.k, w.kh))
        torch.cuda.synchronize()
        close(got[b], out.cpu().numpy()[0], f"row {b} batched vs alone")


@pytest.mark.parametrize("case", ["same_sets", "disjoint", "no_neurons", "no_heads", "all"])
def test_batched_edge_cases(dv, host_layers, case):
    w = W_RAG16
    t = host_layers[w.name]
    B = 8
    rng = np.random.default_rng(5)
    x = synth.x_input(w.with_(batch=B), step=4)
    if case == "same_sets":
        S = np.repeat(random_sets(rng, 1, w.d_ffn, w.k), B, 0)
        Sh = np.repeat(random_sets(rng, 1, w.n_heads, w.kh), B, 0)
    elif case == "disjoint":
        perm = rng.permutation(w.d_ffn)[: B * 50].reshape(B, 50)   # 8 rows x 50 neurons, no overlap
        S = np.sort(perm, 1).astype(np.int32)
        Sh = np.stack([np.array([b % w.n_heads]) for b in range(B)]).astype(np.int32)
    elif case == "no_neurons":
        S = np.zeros((B, 0), np.int32)
        Sh = random_sets(rng, B, w.n_heads, w.kh)
    elif case == "no_heads":
        S = random_sets(rng, B, w.d_ffn, w.k)
        Sh = np.zeros((B, 0), np.int32)
    else:
        S = np.tile(np.arange(w.d_ffn, dtype=np.int32), (B, 1))
        Sh = np.tile(np.arange(w.n_heads, dtype=np.int32), (B, 1))
    got, *_ = run_layer(dv, w, t, x, S, Sh)
    wc = w.with_(batch=B)
    ref = oracle.layer(x, t, kv_host(wc, "k_cache"), kv_host(wc, "v_cache"), w.t_past, S, Sh)
    close(got, ref["out"], f"{case} layer out")
    if S.shape[1] > 0:
        close(got - ref["h1"], ref["y_m"], f"{case} y_m")


@pytest.mark.parametrize("B", [8, 17])
def test_batched_deterministic(dv, host_layers, B):
    """Two runs give the same bits: at B = 8 the up-projections split K on the device (the
    slice count follows the union's device-side size), at B = 17 they do not."""
    w = W_C2
    t = host_layers[w.name]
    x = synth.x_input(w.with_(batch=B), step=8)
    S = zipf_sets(w, B, w.d_ffn, w.k, "sel_mlp")
    Sh = zipf_sets(w, B, w.n_heads, w.kh, "sel_head")
    a, *_ = run_layer(dv, w, t, x, S, Sh)
    b, *_ = run_layer(dv, w, t, x, S, Sh)
    assert np.array_equal(a, b), "batched step must be bitwise reproducible"


@pytest.mark.parametrize("B", [2, 8, 17, 32])
def test_batched_predictor(dv, host_layers, B):
    w = W_C2
    t = host_layers[w.name]
    x = synth.x_input(w.with_(batch=B), step=6)
    d = to_dev({**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")}, "x": x})
    dims = dims_of(w)
    s_m = torch.empty(B, w.d_ffn, device="cuda")
    s_h = torch.empty(B, w.n_heads, device="cuda")
    dv.dv_predict(dims, pred_weights(d), d["x"], s_m, s_h, dv.workspace(dims, B, w.k, w.kh))
    torch.cuda.synchronize()
    rm, rh = oracle.predict(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"], x)
    # split products keep the single-row bar (rel 1e-3) on the batched path
    assert_scores_close(s_m.cpu().numpy(), rm, "s_mlp")
    assert_scores_close(s_h.cpu().numpy(), rh, "s_head")


def test_batched_stack_two_streams_equal_serial(dv):
    """Lookahead stack at B = 8 (union path): the side-stream schedule gives the same bits as
    serial execution, and every layer matches the oracle's own stack (its sets equal the
    GPU's, or differ only at near ties)."""
    w = W_RAG16.with_(batch=8)
    n = 2
    host = [synth.layer_tensors(w, l) for l in range(n)]
    dev = [to_dev(h) for h in host]
    kcs = [kv_host(w, "k_cache", l) for l in range(n)]
    vcs = [kv_host(w, "v_cache", l) for l in range(n)]
    x = synth.x_input(w, step=2)
    dims = dims_of(w)

    def run(two):
        kcd = [torch.from_numpy(a).cuda() for a in kcs]
        vcd = [torch.from_numpy(a).cuda() for a in vcs]
        xd = torch.from_numpy(x).cuda()
        y = torch.empty_like(xd)
        h_all = torch.empty(n + 1, w.batch, w.d_model, device="cuda")
        io = torch.empty(n, w.batch, w.k, dtype=torch.int32, device="cuda")
        ho = torch.empty(n, w.batch, w.kh, dtype=torch.int32, device="cuda")
        ws = dv.stack_workspace(dims, w.batch, w.k, w.kh)
        dv.dv_lookahead_stack(dims, [layer_weights(t) for t in dev], [pred_weights(t) for t in dev], xd, w.k, w.kh,
                              kcd, vcd, w.t_past, y, h_all=h_all, idx_out=io, heads_out=ho, ws=ws,
                              side_stream=torch.cuda.Stream() if two else None)
        torch.cuda.synchronize()
        return h_all.cpu().numpy(), io.cpu().numpy(), ho.cpu().numpy()

    h2, io2, ho2 = run(True)
    h1, io1, ho1 = run(False)
    assert np.array_equal(h2, h1) and np.array_equal(io2, io1) and np.array_equal(ho2, ho1)
    # the oracle's own stack (its own scores, sets and outputs)
    h_or = [x.astype(np.float64)]
    for l in range(n):
        rm, rh = oracle.predict(host[l]["p1_mlp"], host[l]["p2_mlp"], host[l]["p1_head"], host[l]["p2_head"],
                                h_or[max(l - 1, 0)])
        S = chosen_sets(io2[l], rm, w.k, f"layer {l} neuron sets")
        Sh = chosen_sets(ho2[l], rh, w.kh, f"layer {l} head sets")
        ref = oracle.layer(h_or[l], host[l], kcs[l], vcs[l], w.t_past, S, Sh)
        close(h2[l + 1], ref["out"], f"layer {l} output", bar=BATCHED_BAR * (l + 1))
        h_or.append(ref["out"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("B", [8, 32])
def test_opt175b_batched_full_size_sampled_rows(dv, B):
    """The OPT-175B-shaped layer at B = 8 (up-projections split K on the device) and B = 32
    (KV 1024, Zipf selections) on the union path, in the launch configuration the batched
    bench times; three sampled rows checked against the oracle on their regenerated selected
    rows (output, MLP part and the appended k/v), and the batched predictor's scores of those
    rows against the oracle's."""
    import synth.device as sdev
    from helpers import oracle_layer_compact, predictor_host
    w = synth.OPT175B_BATCHED.with_(batch=B)
    B = w.batch
    dims = dims_of(w)
    t = sdev.layer_on_device(w, 0)
    kc = sdev.kv_on_device(w, "k_cache", 0)
    vc = sdev.kv_on_device(w, "v_cache", 0)
    S = zipf_sets(w, B, w.d_ffn, w.k, "sel_mlp")
    Sh = zipf_sets(w, B, w.n_heads, w.kh, "sel_head")
    x = synth.x_input(w, step=5)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    s_m = torch.empty(B, w.d_ffn, device="cuda")
    s_h = torch.empty(B, w.n_heads, device="cuda")
    ws = dv.workspace(dims, B, w.k, w.kh)
    dv.dv_predict(dims, pred_weights(t), xd, s_m, s_h, ws)
    dv.dv_layer_step(dims, layer_weights(t), None, xd, None, w.k, w.kh, torch.from_numpy(S).cuda(),
                     torch.from_numpy(Sh).cuda(), kc, vc, w.t_past, out, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gm, gh = s_m.cpu().numpy(), s_h.cpu().numpy()
    rows = (0, B // 2 - 3, B - 1)
    p = predictor_host(w, 0)
    rm, rh = oracle.predict(p["p1_mlp"], p["p2_mlp"], p["p1_head"], p["p2_head"], x[list(rows)])
    assert_scores_close(gm[list(rows)], rm, "full-size s_mlp")
    assert_scores_close(gh[list(rows)], rh, "full-size s_head")
    for b in rows:
        ref = oracle_layer_compact(w, 0, x[b], S[b], Sh[b], b)
        close(got[b:b + 1], ref["out"], f"row {b} layer out")
        close(got[b:b + 1] - ref["h1"], ref["y_m"], f"row {b} y_m")
        for j, h in enumerate(Sh[b]):
            for m, cache in ((1, kc), (2, vc)):
                slot = cache[b, h, w.t_past].float().cpu().numpy().astype(np.float64)
                r = ref["qkv"][0, j, m]
                assert np.max(np.abs(slot - r)) <= BATCHED_BAR * 4 * max(rms(r), 1e-30) + 2 ** -10 * np.max(np.abs(r))
    del t, kc, vc, ws
    torch.cuda.empty_cache()

@pytest.mark.timeout(900)
def test_opt175b_batched_every_neuron_two_row_sweeps(dv):
    """The OPT-175B-shaped layer at B = 3 with every neuron selected: the union holds all
    49152 neurons, so each row group of the down-projection spans 3072 union positions and
    its weight-row numbers are staged in LDS in two sweeps (2048, then 1024 positions); the
    up-projections split K on the device over 768 tiles. Row 1 is checked against the oracle
    on its regenerated rows (output and MLP part)."""
    import synth.device as sdev
    from helpers import oracle_layer_compact
    w = synth.OPT175B_BATCHED.with_(batch=3, k=49152)
    B = w.batch
    dims = dims_of(w)
    t = sdev.layer_on_device(w, 0)
    kc = sdev.kv_on_device(w, "k_cache", 0)
    vc = sdev.kv_on_device(w, "v_cache", 0)
    S = np.tile(np.arange(w.d_ffn, dtype=np.int32), (B, 1))
    Sh = zipf_sets(w, B, w.n_heads, w.kh, "sel_head")
    x = synth.x_input(w, step=2)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    ws = dv.workspace(dims, B, w.k, w.kh)
    dv.dv_layer_step(dims, layer_weights(t), None, xd, None, w.k, w.kh, torch.from_numpy(S).cuda(),
                     torch.from_numpy(Sh).cuda(), kc, vc, w.t_past, out, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del t, kc, vc, ws
    torch.cuda.empty_cache()
    b = 1
    ref = oracle_layer_compact(w, 0, x[b], S[b], Sh[b], b)
    close(got[b:b + 1], ref["out"], f"row {b} layer out")
    close(got[b:b + 1] - ref["h1"], ref["y_m"], f"row {b} y_m")
