"""Full-size shapes in the launch configurations the bench times (GPU), checked against the
oracle on the regenerated selected rows (the compacted oracle equals the masked dense oracle,
pinned on the CPU):

* the OPT-66B-shaped layer (d 9216, F 36864, 72 x 128 heads, KV 2048, rank 1000) with sets
  predicted inline at three density points of the sweep, including every head and neuron;
* three consecutive decode tokens through two OPT-175B-shaped layers (d 12288, F 49152,
  96 x 128 heads, rank 1000) with the past length held per row in device memory and advanced
  by the call, against the oracle's own decode (its own scores, sets, outputs and caches);
  the same at B = 8 with ragged lengths on the union path (two tokens, three sampled rows).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from helpers import (FP16_BAR, assert_close, assert_scores_close, chosen_sets, dims_of, layer_weights,
                     oracle_layer_compact, pred_weights, predictor_host, rms)

pytestmark = pytest.mark.gpu


def appended_ok(slot, ref):
    """A k or v appended in fp16 against the oracle's fp64 value: the storage rounding
    (2^-11 relative, taken as 2^-10 of the row's largest magnitude) plus the layer bar."""
    slot = np.asarray(slot, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(slot - ref))) <= 2.0 ** -10 * float(np.max(np.abs(ref))) + FP16_BAR * max(rms(ref), 1e-30)


W66 = synth.OPT66B_LAYER
CELLS = [(0.05, 0.20), (0.02, 0.10), (1.00, 1.00)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mlp,head", CELLS, ids=[f"mlp{int(m * 100)}-head{int(h * 100)}" for m, h in CELLS])
def test_opt66b_shape_inline_prediction(dv, mlp, head):
    w = W66.with_(k=synth.count_at(mlp, W66.d_ffn), kh=synth.count_at(head, W66.n_heads))
    dims = dims_of(w)
    t = sdev.layer_on_device(w, 0)
    kc = sdev.kv_on_device(w, "k_cache", 0)
    vc = sdev.kv_on_device(w, "v_cache", 0)
    x = synth.x_input(w, step=3)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    io = torch.empty(1, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(1, w.kh, dtype=torch.int32, device="cuda")
    s_m = torch.empty(1, w.d_ffn, device="cuda")
    s_h = torch.empty(1, w.n_heads, device="cuda")
    ws = dv.workspace(dims, 1, w.k, w.kh)
    dv.dv_predict(dims, pred_weights(t), xd, s_m, s_h, ws)
    tm = torch.empty(1, w.k, dtype=torch.int32, device="cuda")
    th = torch.empty(1, w.kh, dtype=torch.int32, device="cuda")
    dv.dv_topk(s_m, w.k, tm)
    dv.dv_topk(s_h, w.kh, th)
    dv.dv_layer_step(dims, layer_weights(t), pred_weights(t), xd, xd, w.k, w.kh, None, None, kc, vc, w.t_past, out,
                     io, ho, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    S_gpu, Sh_gpu = io.cpu().numpy(), ho.cpu().numpy()
    # inside the library the sets are the top-k of its own scores
    assert np.array_equal(S_gpu, tm.cpu().numpy()) and np.array_equal(Sh_gpu, th.cpu().numpy())
    # against the oracle's own prediction and selection
    p = predictor_host(w, 0)
    rm, rh = oracle.predict(p["p1_mlp"], p["p2_mlp"], p["p1_head"], p["p2_head"], x)
    assert_scores_close(s_m.cpu().numpy(), rm, "s_mlp")
    assert_scores_close(s_h.cpu().numpy(), rh, "s_head")
    S = chosen_sets(S_gpu, rm, w.k, "neuron set")[0]
    Sh = chosen_sets(Sh_gpu, rh, w.kh, "head set")[0]
    ref = oracle_layer_compact(w, 0, x[0], S, Sh, 0)
    assert_close(got, ref["out"], w.dtype, "layer out")
    assert_close(got - ref["h1"], ref["y_m"], w.dtype, "y_m")
    # the appended k/v of the selected heads; unselected heads leave slot T untouched (zero)
    kch = kc[0, :, w.t_past].float().cpu().numpy()
    vch = vc[0, :, w.t_past].float().cpu().numpy()
    for j, h in enumerate(Sh):
        assert appended_ok(kch[h], ref["qkv"][0, j, 1]), f"appended k of head {h}"
        assert appended_ok(vch[h], ref["qkv"][0, j, 2]), f"appended v of head {h}"
    others = np.setdiff1d(np.arange(w.n_heads), Sh)
    assert not kch[others].any() and not vch[others].any(), "an unselected head wrote its slot"
    # the attention block alone (y_a) on the oracle's normalised input, fresh caches
    kc2 = sdev.kv_on_device(w, "k_cache", 0)
    vc2 = sdev.kv_on_device(w, "v_cache", 0)
    ya = torch.empty_like(xd)
    xn = torch.from_numpy(ref["xn1"].astype(np.float32)).cuda()
    dv.dv_sparse_attn(dims, layer_weights(t), xn, torch.from_numpy(Sh[None].astype(np.int32)).cuda(), w.kh, kc2, vc2,
                      w.t_past, ya, ws)
    torch.cuda.synchronize()
    assert_close(ya.cpu().numpy(), ref["y_a"], w.dtype, "y_a")
    del t, kc, vc, kc2, vc2, ws
    torch.cuda.empty_cache()


W175 = synth.OPT175B_STACK
TOKENS = 3


def decode_cache_rows(wd, which, layer, heads, t0, appended):
    """Row 0's cache of the given heads [1][len(heads)][t_max][dh]: the seeded past (slots
    below t0), the oracle's own appends of earlier tokens, zero elsewhere (holes)."""
    shp = (wd.n_heads, wd.t_max, wd.head_dim)
    r = synth.rows(wd.key(which, layer), shp, wd.kv_sigma, wd.dtype, np.asarray(heads))
    r[:, t0:, :] = 0
    for j, h in enumerate(heads):
        for slot, val in appended.get(int(h), {}).items():
            r[j, slot] = val
    return r[None]


@pytest.mark.timeout(900)
def test_opt175b_shape_decode_three_tokens(dv):
    """dv_decode_step on two OPT-175B-shaped layers for three consecutive tokens (KV 2048 ->
    2050, lengths on the device, advanced by the call, side-stream lookahead)."""
    n = 2
    t0 = W175.t_past
    wd = W175.with_(t_past=t0 + TOKENS - 1)          # t_max = t0 + TOKENS: room for the decode
    dims = dims_of(wd)
    dev = [sdev.layer_on_device(W175, l) for l in range(n)]
    kcd, vcd = [], []
    for l in range(n):
        for which, lst in (("k_cache", kcd), ("v_cache", vcd)):
            c = sdev.kv_on_device(wd, which, l)
            c[:, :, t0:, :] = 0
            lst.append(c)
    t_rows = torch.full((1,), t0, dtype=torch.int32, device="cuda")
    ws = dv.stack_workspace(dims, 1, W175.k, W175.kh)
    side = torch.cuda.Stream()
    preds = [predictor_host(W175, l) for l in range(n)]
    appended = [{"k_cache": {}, "v_cache": {}} for _ in range(n)]   # oracle's own appends: head -> slot -> fp16
    for s in range(TOKENS):
        T = t0 + s
        x = synth.x_input(W175, step=200 + s)
        xd = torch.from_numpy(x).cuda()
        y = torch.empty_like(xd)
        h_all = torch.empty(n + 1, 1, W175.d_model, device="cuda")
        io = torch.empty(n, 1, W175.k, dtype=torch.int32, device="cuda")
        ho = torch.empty(n, 1, W175.kh, dtype=torch.int32, device="cuda")
        dv.dv_decode_step(dims, [layer_weights(t) for t in dev], [pred_weights(t) for t in dev], xd, W175.k, W175.kh,
                          kcd, vcd, t_rows, y, advance=True, h_all=h_all, idx_out=io, heads_out=ho, ws=ws,
                          side_stream=side)
        torch.cuda.synchronize()
        assert int(t_rows.item()) == min(T + 1, wd.t_max - 1)   # the advance saturates at t_max - 1
        h = h_all.cpu().numpy()
        S_all, Sh_all = io.cpu().numpy(), ho.cpu().numpy()
        h_or = [x.astype(np.float64)]
        for l in range(n):
            p = preds[l]
            rm, rh = oracle.predict(p["p1_mlp"], p["p2_mlp"], p["p1_head"], p["p2_head"], h_or[max(l - 1, 0)])
            S = chosen_sets(S_all[l], rm, W175.k, f"token {s} layer {l} neuron set")[0]
            Sh = chosen_sets(Sh_all[l], rh, W175.kh, f"token {s} layer {l} head set")[0]
            tw = _compact_weights(W175, l, S, Sh)
            kc = decode_cache_rows(wd, "k_cache", l, Sh, t0, appended[l]["k_cache"])
            vc = decode_cache_rows(wd, "v_cache", l, Sh, t0, appended[l]["v_cache"])
            ref = oracle.layer(h_or[l], tw, kc, vc, T, [np.arange(len(S))], [np.arange(len(Sh))])
            assert_close(h[l + 1], ref["out"], W175.dtype, f"token {s} layer {l} output", depth=l + 1 + s)
            gk = kcd[l][0, :, T].float().cpu().numpy()
            gv = vcd[l][0, :, T].float().cpu().numpy()
            for j, hd in enumerate(Sh):
                rk, rv = ref["qkv"][0, j, 1], ref["qkv"][0, j, 2]
                assert appended_ok(gk[hd], rk) and appended_ok(gv[hd], rv), f"token {s} layer {l} head {hd} k/v"
                appended[l]["k_cache"].setdefault(int(hd), {})[T] = rk.astype(np.float16)
                appended[l]["v_cache"].setdefault(int(hd), {})[T] = rv.astype(np.float16)
            others = np.setdiff1d(np.arange(W175.n_heads), Sh)
            assert not gk[others].any() and not gv[others].any(), "an unselected head wrote its slot (hole)"
            h_or.append(ref["out"])
    del dev, kcd, vcd, ws
    torch.cuda.empty_cache()


def _row_cache(wd, which, layer, b, heads, t0, appended):
    """Row b's cache of the given heads [1][len(heads)][t_max][dh] for a batch of wd.batch rows:
    the seeded past (slots below the row's own start t0), the oracle's own appends, zero
    elsewhere."""
    shp = (wd.batch * wd.n_heads, wd.t_max, wd.head_dim)
    r = synth.rows(wd.key(which, layer), shp, wd.kv_sigma, wd.dtype, b * wd.n_heads + np.asarray(heads))
    r[:, t0:, :] = 0
    for j, h in enumerate(heads):
        for slot, val in appended.get(int(h), {}).items():
            r[j, slot] = val
    return r[None]


@pytest.mark.timeout(900)
def test_opt175b_shape_decode_batch8_ragged(dv):
    """dv_decode_step on two OPT-175B-shaped layers at B = 8, past lengths 256, 512, ..., 2048
    held per row on the device and advanced by the call, for two consecutive tokens: the union
    path on the matrix cores with the side-stream lookahead, as the multi-step decode bench
    runs it. Rows 0, 3 and 7 against the oracle's own decode of that row (its own scores,
    sets, outputs and caches)."""
    n, B, tokens = 2, 8, 2
    starts = [256 * (b + 1) for b in range(B)]
    wd = W175.with_(batch=B, t_past=max(starts) + tokens)   # t_max = longest start + tokens + 1: no saturation
    dims = dims_of(wd)
    dev = [sdev.layer_on_device(W175, l) for l in range(n)]
    kcd, vcd = [], []
    for l in range(n):
        for which, lst in (("k_cache", kcd), ("v_cache", vcd)):
            c = sdev.kv_on_device(wd, which, l)
            for b, t0 in enumerate(starts):
                c[b, :, t0:, :] = 0
            lst.append(c)
    t_rows = torch.tensor(starts, dtype=torch.int32, device="cuda")
    ws = dv.stack_workspace(dims, B, W175.k, W175.kh)
    side = torch.cuda.Stream()
    preds = [predictor_host(W175, l) for l in range(n)]
    rows = (0, 3, 7)
    appended = {(b, l, which): {} for b in rows for l in range(n) for which in ("k_cache", "v_cache")}
    for s in range(tokens):
        x = synth.x_input(wd, step=300 + s)
        xd = torch.from_numpy(x).cuda()
        y = torch.empty_like(xd)
        h_all = torch.empty(n + 1, B, W175.d_model, device="cuda")
        io = torch.empty(n, B, W175.k, dtype=torch.int32, device="cuda")
        ho = torch.empty(n, B, W175.kh, dtype=torch.int32, device="cuda")
        dv.dv_decode_step(dims, [layer_weights(t) for t in dev], [pred_weights(t) for t in dev], xd, W175.k, W175.kh,
                          kcd, vcd, t_rows, y, advance=True, h_all=h_all, idx_out=io, heads_out=ho, ws=ws,
                          side_stream=side)
        torch.cuda.synchronize()
        assert t_rows.cpu().tolist() == [t0 + s + 1 for t0 in starts]
        h = h_all.cpu().numpy()
        S_all, Sh_all = io.cpu().numpy(), ho.cpu().numpy()
        for b in rows:
            T = starts[b] + s
            h_or = [x[b].astype(np.float64)[None]]
            for l in range(n):
                p = preds[l]
                rm, rh = oracle.predict(p["p1_mlp"], p["p2_mlp"], p["p1_head"], p["p2_head"], h_or[max(l - 1, 0)])
                S = chosen_sets(S_all[l][b:b + 1], rm, W175.k, f"token {s} row {b} layer {l} neuron set")[0]
                Sh = chosen_sets(Sh_all[l][b:b + 1], rh, W175.kh, f"token {s} row {b} layer {l} head set")[0]
                tw = _compact_weights(W175, l, S, Sh)
                kc = _row_cache(wd, "k_cache", l, b, Sh, starts[b], appended[(b, l, "k_cache")])
                vc = _row_cache(wd, "v_cache", l, b, Sh, starts[b], appended[(b, l, "v_cache")])
                ref = oracle.layer(h_or[l], tw, kc, vc, T, [np.arange(len(S))], [np.arange(len(Sh))])
                assert_close(h[l + 1][b:b + 1], ref["out"], W175.dtype, f"token {s} row {b} (T={T}) layer {l}",
                             batch=B, depth=l + 1 + s)
                gk = kcd[l][b, :, T].float().cpu().numpy()
                gv = vcd[l][b, :, T].float().cpu().numpy()
                for j, hd in enumerate(Sh):
                    rk, rv = ref["qkv"][0, j, 1], ref["qkv"][0, j, 2]
                    assert appended_ok(gk[hd], rk) and appended_ok(gv[hd], rv), f"token {s} row {b} head {hd} k/v"
                    appended[(b, l, "k_cache")].setdefault(int(hd), {})[T] = rk.astype(np.float16)
                    appended[(b, l, "v_cache")].setdefault(int(hd), {})[T] = rv.astype(np.float16)
                others = np.setdiff1d(np.arange(W175.n_heads), Sh)
                assert not gk[others].any() and not gv[others].any(), f"row {b}: an unselected head wrote its slot"
                h_or.append(ref["out"])
    del dev, kcd, vcd, ws
    torch.cuda.empty_cache()


def _compact_weights(w, layer, S, Sh):
    """Selected weight rows of one layer (the weights part of the compacted oracle inputs)."""
    shapes = synth.layer_shapes(w)
    t = {}
    for name in ("wqkv", "bqkv", "wo"):
        shp, sg, dt = shapes[name]
        t[name] = synth.rows(w.key(name, layer), shp, sg, dt, Sh)
    for name in ("w1t", "b1", "w2"):
        shp, sg, dt = shapes[name]
        t[name] = synth.rows(w.key(name, layer), shp, sg, dt, S)
    for name in ("bo", "b2"):
        shp, sg, dt = shapes[name]
        t[name] = synth.tensor(w.key(name, layer), shp, sg, dt)
    t["g1"] = synth.gains(w)
    t["g2"] = synth.gains(w)
    return t
