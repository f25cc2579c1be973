"""Lookahead stack: the GPU stack against the oracle running the same stack on its own
(its own scores, sets and layer outputs, nothing taken from the GPU), two streams == one
stream bitwise, and the OPT-175B-shaped layer at full size in the launch configuration the
bench times (GPU). The GPU's sets must equal the oracle's, or differ only at near ties of the
oracle's scores (then the oracle continues with the GPU's equally correct choice)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from helpers import (W_C2, W_RAG16, assert_close, chosen_sets, dims_of, kv_host, layer_weights,
                     oracle_layer_compact, pred_weights, predictor_host, to_dev)

pytestmark = pytest.mark.gpu


def build_stack(w, n_layers):
    host = [synth.layer_tensors(w, l) for l in range(n_layers)]
    dev = [to_dev(t) for t in host]
    kcs = [kv_host(w, "k_cache", l) for l in range(n_layers)]
    vcs = [kv_host(w, "v_cache", l) for l in range(n_layers)]
    return host, dev, kcs, vcs


def run_stack(dv, w, dev, kcs, vcs, x, two_streams):
    n = len(dev)
    dims = dims_of(w)
    kcd = [torch.from_numpy(a).cuda() for a in kcs]
    vcd = [torch.from_numpy(a).cuda() for a in vcs]
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    h_all = torch.empty(n + 1, w.batch, w.d_model, device="cuda")
    io = torch.empty(n, w.batch, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(n, w.batch, w.kh, dtype=torch.int32, device="cuda")
    ws = dv.stack_workspace(dims, w.batch, w.k, w.kh)
    side = torch.cuda.Stream() if two_streams else None
    dv.dv_lookahead_stack(dims, [layer_weights(t) for t in dev], [pred_weights(t) for t in dev], xd, w.k, w.kh,
                          kcd, vcd, w.t_past, y, h_all=h_all, idx_out=io, heads_out=ho, ws=ws, side_stream=side)
    torch.cuda.synchronize()
    return y.cpu().numpy(), h_all.cpu().numpy(), io.cpu().numpy(), ho.cpu().numpy()


@pytest.mark.parametrize("w", [W_C2.with_(t_past=300), W_RAG16], ids=["opt6.7b-shape", "ragged"])
def test_stack_against_oracle_stack_and_stream_invariant(dv, w):
    n = 3
    host, dev, kcs, vcs = build_stack(w, n)
    x = synth.x_input(w, step=2)
    y2, h2, io2, ho2 = run_stack(dv, w, dev, kcs, vcs, x, two_streams=True)
    y1, h1, io1, ho1 = run_stack(dv, w, dev, kcs, vcs, x, two_streams=False)
    assert np.array_equal(h2, h1) and np.array_equal(io2, io1) and np.array_equal(ho2, ho1), \
        "side-stream lookahead must give the same bits as serial execution"
    assert np.array_equal(y2, h2[n]) and np.array_equal(h2[0], x)
    # the oracle's own stack: the sets of layer l are the top-k of predictor l applied to
    # the input of layer l-1 (layer 0: the stack input)
    h_or = [x.astype(np.float64)]
    for l in range(n):
        src = h_or[max(l - 1, 0)]
        rm, rh = oracle.predict(host[l]["p1_mlp"], host[l]["p2_mlp"], host[l]["p1_head"], host[l]["p2_head"], src)
        S = chosen_sets(io2[l], rm, w.k, f"layer {l} neuron set")
        Sh = chosen_sets(ho2[l], rh, w.kh, f"layer {l} head set")
        ref = oracle.layer(h_or[l], host[l], kcs[l], vcs[l], w.t_past, S, Sh)
        assert_close(h2[l + 1], ref["out"], w.dtype, f"layer {l} output", depth=l + 1)
        h_or.append(ref["out"])


W175 = synth.OPT175B_STACK


@pytest.mark.timeout(900)
def test_opt175b_shape_full_size_two_layers(dv):
    """Full OPT-175B layer shape (d 12288, F 49152, 96x128 heads, KV 2048, rank 1000, k 2458,
    kh 19) through the same stack driver and tiling as the bench; every output of both
    layers checked against the oracle's own two layers on the regenerated selected rows."""
    w = W175
    n = 2
    dims = dims_of(w)
    dev = [sdev.layer_on_device(w, l) for l in range(n)]
    kcd = [sdev.kv_on_device(w, "k_cache", l) for l in range(n)]
    vcd = [sdev.kv_on_device(w, "v_cache", l) for l in range(n)]
    x = sdev.x_on_device(w, step=0)
    y = torch.empty_like(x)
    h_all = torch.empty(n + 1, 1, w.d_model, device="cuda")
    io = torch.empty(n, 1, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(n, 1, w.kh, dtype=torch.int32, device="cuda")
    ws = dv.stack_workspace(dims, 1, w.k, w.kh)
    side = torch.cuda.Stream()
    dv.dv_lookahead_stack(dims, [layer_weights(t) for t in dev], [pred_weights(t) for t in dev], x, w.k, w.kh,
                          kcd, vcd, w.t_past, y, h_all=h_all, idx_out=io, heads_out=ho, ws=ws, side_stream=side)
    torch.cuda.synchronize()
    h = h_all.cpu().numpy()
    S, Sh = io.cpu().numpy(), ho.cpu().numpy()
    x_host = synth.x_input(w, step=0)
    assert np.array_equal(h[0], x_host)
    # the oracle's own two layers: both layers' sets come from predictors applied to the
    # stack input (layer 1 reads the input of layer 0)
    h_or = [x_host.astype(np.float64)]
    for l in range(n):
        p = predictor_host(w, l)
        rm, rh = oracle.predict(p["p1_mlp"], p["p2_mlp"], p["p1_head"], p["p2_head"], h_or[max(l - 1, 0)])
        Sl = chosen_sets(S[l], rm, w.k, f"layer {l} neuron set")
        Shl = chosen_sets(Sh[l], rh, w.kh, f"layer {l} head set")
        ref = oracle_layer_compact(w, l, h_or[l][0], Sl[0], Shl[0], 0)
        assert_close(h[l + 1], ref["out"], w.dtype, f"layer {l} output", depth=l + 1)
        if l == 0:   # identical inputs: the MLP part on its own scale
            assert_close(h[1] - ref["h1"], ref["y_m"], w.dtype, "layer 0 y_m")
        h_or.append(ref["out"])
    del dev, kcd, vcd
    torch.cuda.empty_cache()


def test_device_generator_matches_host(dv):
    for dt, sg in (("f16", 0.02), ("f32", 1.0)):
        key = synth.stream_key(3, 1, 2, 7)
        host = synth.tensor(key, (1000, 37), sg, dt)
        t = torch.empty(1000, 37, dtype=torch.float16 if dt == "f16" else torch.float32, device="cuda")
        sdev.fill_(t, key, sg)
        torch.cuda.synchronize()
        ib = np.uint16 if dt == "f16" else np.uint32
        got = t.cpu().numpy()
        bad = np.nonzero(got.view(ib).reshape(-1) != host.view(ib).reshape(-1))[0]
        if bad.size:
            f32 = synth.normal_f32(key, 0, host.size, sg)
            rows = [(int(i), float(f32[i]), hex(int(host.view(ib).reshape(-1)[i])),
                     hex(int(got.view(ib).reshape(-1)[i]))) for i in bad[:12]]
            raise AssertionError(f"{dt}: {bad.size} elements differ (index, fp32 value, host bits, device bits): "
                                 f"{rows}")
        part = torch.empty(5, 37, dtype=t.dtype, device="cuda")
        sdev.fill_(part, key, sg, start=17 * 37)
        torch.cuda.synchronize()
        assert np.array_equal(part.cpu().numpy(), host[17:22])


def test_stack_from_two_host_threads(dv):
    """Two host threads run the stack at the same time on their own stream pairs (each with
    its own caches and workspace): the stack's fork/join events are per thread, so every
    run gives the bits of the single-threaded run."""
    import threading
    w = W_RAG16
    n = 3
    host, dev, kcs, vcs = build_stack(w, n)
    xs = [synth.x_input(w, step=s) for s in (4, 5)]
    ref = [run_stack(dv, w, dev, kcs, vcs, x, two_streams=True) for x in xs]
    out = [[None] * 3 for _ in xs]
    err = []

    def worker(t):
        try:
            main = torch.cuda.Stream()
            with torch.cuda.stream(main):
                for rep in range(3):
                    out[t][rep] = run_stack(dv, w, dev, kcs, vcs, xs[t], two_streams=True)
        except Exception as e:  # reported below, on the test's thread
            err.append(e)

    th = [threading.Thread(target=worker, args=(t,)) for t in range(len(xs))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not err, err
    for t in range(len(xs)):
        for rep in range(3):
            for a, b in zip(out[t][rep], ref[t]):
                assert np.array_equal(a, b), f"thread {t} run {rep} differs from the single-threaded run"
