#!/usr/bin/env python3
"""Bench of the contextually sparse decode step on one MI355X.

Workload: the OPT-175B-shaped stack of 24 decoder layers (d 12288, FFN 49152 ReLU,
96 heads x 128, KV 2048 per layer, fp16 weights, predictor rank 1000), batch 1, 5 % of the
neurons (2458) and 20 % of the heads (19) per layer, sets of layer l+1 predicted from the
input of layer l on a side stream while layer l runs. Weights, caches and inputs are
seeded synthetic draws generated in HBM (no trained weights exist here); x is fresh every
step and residual-propagated through the stack.

One step = one token through all 24 layers. Prints one JSON line:
  value = us per sparse decode layer-token (lower is better), plus achieved HBM GB/s on the
  step's algorithmic bytes, the roofline of the q/k/v gather kernel (timed live with HIP
  events on its own stream), the dense layer through the same kernels and through torch,
  and the CPU fp64 oracle timed on one layer-token of the same shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "rowdot_qkv_opt175b_stack24_hbm_traffic.txt")


def source_text(spec: str) -> bytes:
    """Bytes of a source file, or of the part of it between two marker lines when the spec
    reads "path#first marker#next marker" (the marker of the following section ends it)."""
    path, *marks = spec.split("#")
    data = open(os.path.join(HERE, path), "rb").read()
    if marks:
        start = data.index(marks[0].encode())
        end = data.index(marks[1].encode(), start)
        data = data[start:end]
    return data


def measured_traffic(log):
    """HBM bytes per q/k/v gather launch from the committed FETCH_SIZE/WRITE_SIZE counter
    summary (scaled by a plain copy's counter reading), or None when that summary is missing
    or was taken on kernel sources other than the ones in this tree."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_FILE) if l.startswith("traffic_json "))
        rec = json.loads(line[len("traffic_json "):])
        h = hashlib.sha256()
        for src in rec["sources"]:
            h.update(source_text(src))
    except (OSError, StopIteration, ValueError, KeyError) as e:
        log(f"[bench] no usable traffic summary ({e!r}); traffic = null")
        return None
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        log("[bench] the q/k/v kernel changed since its counters were taken; traffic = null")
        return None
    return int(rec["bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true", help="run the predictor on the main stream")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--batch-sizes", default="1,2,4,8,16,32",
                    help="batch sizes of --workload batched (comma-separated, each 1..32)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--shape", choices=["opt6.7b", "opt125m"], default="opt6.7b",
                    help="layer shape of --workload layer")
    ap.add_argument("--layer-steps", type=int, default=1000, help="timed steps of --workload layer")
    ap.add_argument("--sweep-cells", default="",
                    help="cells of --workload sweep as mlp:head densities, comma-separated (default: all 24)")
    ap.add_argument("--sweep-layers", type=int, default=8,
                    help="layers of the lookahead stack that --workload sweep times beside the serial step")
    ap.add_argument("--workload", choices=["stack", "layer", "batched", "sweep", "blocked", "decode", "train"],
                    default="stack",
                    help="stack: the 24-layer OPT-175B-shaped decode step (default); layer: one "
                         "OPT-6.7B-shaped (or, with --shape opt125m, OPT-125m-shaped) layer, 1000 flushed steps "
                         "with fresh x; batched: one "
                         "OPT-175B-shaped layer at batch 1..32 with Zipf-skewed selections; sweep: the "
                         "OPT-66B-shaped layer over MLP x head densities; blocked: per-neuron vs "
                         "32/64-neuron block selection of the OPT-175B-shaped MLP; decode: consecutive "
                         "tokens through the 24-layer stack with a growing KV (one graph per token); train: "
                         "predictor training and recall on the OPT-125m-shaped layer")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import contextual_activation_sparsity_amd as dv
    from contextual_activation_sparsity_amd import _lib, traffic
    import synth
    import synth.device as sdev

    dv.require_gpu()
    if args.workload != "stack":
        out = {"layer": run_layer, "batched": run_batched, "sweep": run_sweep, "blocked": run_blocked,
               "decode": run_decode, "train": run_train}[args.workload](args, log)
        print(json.dumps(out), flush=True)
        return 0
    w = synth.OPT175B_STACK.with_(n_layers=args.layers)
    L = w.n_layers
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t0 = time.time()
    layers, preds, kcs, vcs = [], [], [], []
    for l in range(L):
        t = sdev.layer_on_device(w, l)
        layers.append(dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1",
                                                             "w2", "b2")}))
        preds.append(dv.PredictorWeights(**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")}))
        kcs.append(sdev.kv_on_device(w, "k_cache", l))
        vcs.append(sdev.kv_on_device(w, "v_cache", l))
    n_steps = args.warmup + args.steps
    xs = torch.empty(n_steps, 1, w.d_model, device="cuda")
    for i in range(n_steps):
        sdev.fill_(xs[i], w.key("x", 0, i), w.x_sigma)
    y = torch.empty(1, w.d_model, device="cuda")
    ws = dv.stack_workspace(dims, 1, w.k, w.kh)
    side = None if args.serial else torch.cuda.Stream()
    torch.cuda.synchronize()
    log(f"[bench] {L} layers drawn in HBM in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 1e9:.1f} GB allocated)")

    def step(i):
        dv.dv_lookahead_stack(dims, layers, preds, xs[i], w.k, w.kh, kcs, vcs, w.t_past, y, ws=ws,
                              side_stream=side)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)   # 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy of 1 GiB done")

    def timed(run_step, n):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        h0 = time.perf_counter()
        for i in range(n):
            run_step(args.warmup + i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n, (time.perf_counter() - h0) * 1e3 / n

    # (1) eager launches, no instrumentation
    ms_eager, wall_eager = timed(step, args.steps)
    log(f"[bench] eager: {ms_eager:.3f} ms/step ({ms_eager * 1e3 / L:.2f} us/layer-token, host {wall_eager:.3f} ms)")

    # (2) the whole two-stream step captured once in a HIP graph and replayed (fresh x is
    #     copied into the graph's input buffer before each replay)
    ms_graph = None
    step_dist = None
    if not args.no_graph:
        x_in = torch.empty(1, w.d_model, device="cuda")
        x_in.copy_(xs[0])
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dv.dv_lookahead_stack(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, w.t_past, y, ws=ws,
                                  side_stream=side)
        torch.cuda.synchronize()

        def gstep(i):
            x_in.copy_(xs[i])
            graph.replay()
        for i in range(3):
            gstep(i)
        ms_graph, wall_graph = timed(gstep, args.steps)
        log(f"[bench] graph: {ms_graph:.3f} ms/step ({ms_graph * 1e3 / L:.2f} us/layer-token, host {wall_graph:.3f} ms)")
        # distribution: replays timed one by one (synchronised in between; not the headline)
        per = []
        for i in range(min(50, args.steps)):
            x_in.copy_(xs[args.warmup + i])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / L)
        step_dist = {"p10": round(float(np.percentile(per, 10)), 3), "p50": round(float(np.median(per)), 3),
                     "p90": round(float(np.percentile(per, 90)), 3), "replays": len(per)}
        log(f"[bench] per-replay us/layer-token: {step_dist}")

    # (2b) where the time goes, each as a captured graph replayed back to back: the layers alone
    #      with their sets given (the main chain), the predictions alone (the side chain: both
    #      stage-1 factors, stage 2 and the top-k of every layer), and the whole step with the
    #      predictions on the main stream (serial)
    split = None
    if not args.no_graph:
        split = time_split(dv, w, dims, layers, preds, kcs, vcs, xs, ws, y, args, log)

    # (3) eager again with HIP event pairs around every q/k/v gather launch (on its stream)
    n_ev = args.steps * L
    assert _lib.lib().dv_timing_start(n_ev) == n_ev
    ms_hooked, _ = timed(step, args.steps)
    import ctypes
    qkv_ms = (ctypes.c_float * n_ev)()
    got = _lib.lib().dv_timing_stop(qkv_ms, n_ev)
    assert got == n_ev, f"timing hook recorded {got} of {n_ev}"
    qkv_ms = np.array(qkv_ms[:n_ev], dtype=np.float64)
    log(f"[bench] instrumented eager pass: {ms_hooked:.3f} ms/step")

    # plain streaming read on the same GPU (4 GiB, every byte loaded once), best of 5: the
    # reference a read-only kernel reaches here, reported beside the 8 TB/s peak
    stream_read = sdev.stream_read_gbps()
    log(f"[bench] plain streaming read: {stream_read:.0f} GB/s")

    ms_per_step = ms_graph if ms_graph is not None else ms_eager
    us_per_layer = ms_per_step * 1e3 / L

    tb = traffic.step_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.t_past, w.k, w.kh, 2)
    step_bytes = tb["total"]
    gbps = step_bytes / (us_per_layer * 1e-6) / 1e9
    # q/k/v gather launch: weight rows + biases of the selected heads, input x, gains, q/k/v
    # out; in layers 0..L-2 the next layer's predictor stage 1 (both rank-r factors over the
    # same x, z out) rides in the same launch.
    d, dh, kh, r = w.d_model, w.head_dim, w.kh, w.rank
    qkv_bytes = 3 * kh * dh * d * 2 + 3 * kh * dh * 4 + d * 4 + d * 4 + 3 * kh * dh * 4 + kh * 4
    p1_bytes = 2 * r * d * 2 + 2 * r * 4
    launch_bytes = np.array([qkv_bytes + (p1_bytes if l + 1 < L else 0) for l in range(L)] * args.steps,
                            dtype=np.float64)
    qkv_avg_us = float(np.mean(qkv_ms)) * 1e3
    qkv_gbps = float(launch_bytes.sum()) / (float(qkv_ms.sum()) * 1e-3) / 1e9

    out = {
        "metric": "µs per sparse decode layer-token + achieved HBM GB/s (% of peak), OPT-175B shape",
        "value": round(us_per_layer, 3),
        "unit": "us/layer-token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "opt175b-shaped 24-layer sparse decode stack, lookahead predictor on a side stream",
                   "layers": L, "d_model": w.d_model, "d_ffn": w.d_ffn, "n_heads": w.n_heads,
                   "head_dim": w.head_dim, "kv_len": w.t_past, "rank": w.rank, "k": w.k, "kh": w.kh,
                   "batch": 1, "storage": "f16 weights and KV, fp32 activations and accumulation",
                   "side_stream": not args.serial,
                   "launch": "hip graph replay" if ms_graph is not None else "eager"},
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": round(ms_graph, 4) if ms_graph is not None else None,
        "achieved_GBps": round(gbps, 1),
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_layer_token": int(step_bytes),
        "bytes_breakdown": {k: int(v) for k, v in tb.items()},
        "roofline": {"bound": "hbm", "achieved": round(qkv_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(qkv_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(log),
                     "kernel": "rowdot_kernel<f16,256,6,qkv>: head-sparse q/k/v gather-GEMV + next layer's "
                               "predictor stage 1",
                     "bytes_per_launch": int(round(launch_bytes.mean())), "avg_launch_us": round(qkv_avg_us, 3),
                     "launches_timed": int(n_ev), "stream_read_GBps": round(stream_read, 1),
                     "frac_of_stream_read": round(qkv_gbps / stream_read, 4)},
        "us_per_layer_token_per_replay": step_dist,
        "time_split_us_per_layer_token": split,
        "step_pct_of_stream_read": round(100.0 * gbps / stream_read, 2),
    }

    if not args.no_dense:
        out["dense"] = dense_baselines(dv, w, dims, layers, kcs, vcs, xs, args.dense_steps, log)
        best = min(v["us_per_layer_token"] for v in out["dense"].values())
        out["speedup_vs_dense"] = round(best / us_per_layer, 3)

    del layers, preds, kcs, vcs, xs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, log)
    print(json.dumps(out), flush=True)
    return 0


def time_split(dv, w, dims, layers, preds, kcs, vcs, xs, ws, y, args, log):
    """Per layer-token: the main chain alone (every layer's sets given, taken from one stack
    run), the side chain alone (predictor and top-k of every layer), the serial step (one
    stream) and the two-stream step, each captured once and replayed back to back."""
    import torch
    L = len(layers)
    io = torch.empty(L, 1, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(L, 1, w.kh, dtype=torch.int32, device="cuda")
    x_in = torch.empty(1, w.d_model, device="cuda")
    x_in.copy_(xs[0])
    dv.dv_lookahead_stack(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, w.t_past, y, idx_out=io, heads_out=ho,
                          ws=ws)
    lws = dv.workspace(dims, 1, w.k, w.kh)
    h = torch.empty(1, w.d_model, device="cuda")
    s_m = torch.empty(1, w.d_ffn, device="cuda")
    s_h = torch.empty(1, w.n_heads, device="cuda")
    pi = torch.empty(1, w.k, dtype=torch.int32, device="cuda")
    ph = torch.empty(1, w.kh, dtype=torch.int32, device="cuda")
    tws_m = torch.empty(dv.dv_topk_workspace_bytes(1, w.d_ffn), dtype=torch.uint8, device="cuda")
    tws_h = torch.empty(dv.dv_topk_workspace_bytes(1, w.n_heads), dtype=torch.uint8, device="cuda")

    def main_chain():
        h.copy_(x_in)
        for l in range(L):
            dv.dv_layer_step(dims, layers[l], None, h, None, w.k, w.kh, io[l], ho[l], kcs[l], vcs[l], w.t_past, h,
                             ws=lws)

    def side_chain():
        for l in range(L):
            dv.dv_predict(dims, preds[l], x_in, s_m, s_h, lws)
            dv.dv_topk(s_m, w.k, pi, tws_m)
            dv.dv_topk(s_h, w.kh, ph, tws_h)

    def serial():
        dv.dv_lookahead_stack(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, w.t_past, y, ws=ws)

    side = torch.cuda.Stream()

    def two_stream():
        dv.dv_lookahead_stack(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, w.t_past, y, ws=ws, side_stream=side)

    out = {}
    n = max(20, min(args.steps, 100))
    for name, fn in (("main_chain_alone", main_chain), ("side_chain_alone", side_chain), ("serial", serial),
                     ("two_streams", two_stream)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / n / L, 2)
        del g
    log(f"[bench] time split (us per layer-token): {out}")
    del lws, tws_m, tws_h
    return out


def dense_baselines(dv, w, dims, layers, kcs, vcs, xs, n_steps, log):
    """The dense layer at the same shape: (a) the library's own gather kernels with every
    neuron and head selected, (b) torch (hipBLASLt F.linear, matmul attention)."""
    import torch
    import torch.nn.functional as Fn
    L = len(layers)
    res = {}
    idx = torch.arange(w.d_ffn, dtype=torch.int32, device="cuda")[None].contiguous()
    heads = torch.arange(w.n_heads, dtype=torch.int32, device="cuda")[None].contiguous()
    ws = dv.workspace(dims, 1, w.d_ffn, w.n_heads)
    h = torch.empty(1, w.d_model, device="cuda")

    def lib_step(x):
        h.copy_(x)
        for l in range(L):
            dv.dv_layer_step(dims, layers[l], None, h, None, w.d_ffn, w.n_heads, idx, heads, kcs[l], vcs[l],
                             w.t_past, h, ws=ws)

    lib_step(xs[0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_steps):
        lib_step(xs[i])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_steps * L)
    res["library_all_selected"] = {"us_per_layer_token": round(us, 2)}
    log(f"[bench] dense through the library: {us:.1f} us/layer-token")

    # torch baseline on layer 0 repeated (its transposed copies exist once); at 3.7 GB per
    # layer nothing stays in cache between repeats.
    torch_full = torch_dense_layer(w, layers[0], kcs[0], vcs[0], 1)
    reps = max(4, n_steps * 2)
    x = xs[0].clone()
    torch_full(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch_full(x)
    e1.record()
    torch.cuda.synchronize()
    us_t = e0.elapsed_time(e1) * 1e3 / reps
    res["torch_dense_layer"] = {"us_per_layer_token": round(us_t, 2),
                                "note": "F.linear (hipBLASLt) projections + bmm attention, fp16 storage"}
    log(f"[bench] dense torch layer: {us_t:.1f} us/layer-token")
    del torch_full
    return res


def torch_dense_layer(w, lw, kc, vc, B):
    """The dense layer in torch for B rows, as a timing comparator: RMSNorm, F.linear
    (hipBLASLt) projections on the storage type with fp32 results, decode attention by bmm over
    each row's T past slots and the current token (written to slot T first, as the sparse step
    appends it; the caches hold t_max = T + 1 slots), ReLU MLP. The transposed copies torch's
    dense form needs for Wo and W2 are made here, once, outside any timed region."""
    import torch
    import torch.nn.functional as Fn
    H, dh, d, T = w.n_heads, w.head_dim, w.d_model, w.t_past
    t_max = kc.shape[2]
    assert t_max == T + 1, "the torch comparator attends over every cache slot"
    st = lw.wqkv.dtype
    wqkv = lw.wqkv.view(H * 3 * dh, d)
    wo_t = lw.wo.view(H * dh, d).t().contiguous()
    w2_t = lw.w2.t().contiguous()
    K = kc[:B].view(B * H, t_max, dh)
    V = vc[:B].view(B * H, t_max, dh)
    scale = 1.0 / dh ** 0.5

    def f(x):
        xn = (x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + 1e-5) * lw.g1).to(st)
        qkv = Fn.linear(xn, wqkv).float().view(B, H, 3, dh) + lw.bqkv
        K[:, T] = qkv[:, :, 1].reshape(B * H, dh).to(st)
        V[:, T] = qkv[:, :, 2].reshape(B * H, dh).to(st)
        q = (qkv[:, :, 0] * scale).reshape(B * H, dh, 1).to(st)
        p = torch.softmax(torch.bmm(K, q).float(), dim=1)                       # [B*H][t_max][1]
        o = torch.bmm(p.transpose(1, 2).to(st).contiguous(), V).float()          # [B*H][1][dh]
        h1 = x + Fn.linear(o.reshape(B, H * dh).to(st), wo_t).float() + lw.bo
        xn2 = (h1 * torch.rsqrt(h1.pow(2).mean(-1, keepdim=True) + 1e-5) * lw.g2).to(st)
        u = torch.relu(Fn.linear(xn2, lw.w1t).float() + lw.b1)
        return h1 + Fn.linear(u.to(st), w2_t).float() + lw.b2

    return f


def timed_single_layer(step, n_steps, log, work=None):
    """Median and 10th/90th percentiles of one step's time (HIP events on the current
    stream), with an untimed 1 GiB write between steps so no weight stays in the 256 MB
    Infinity Cache. `step(i)` records the device work while a graph is being captured and
    otherwise only rotates the inputs; the timed work is then one replay of that graph.
    With `work` given, the timed work is instead the eager call work() (no graph)."""
    import numpy as np
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    if work is None:
        graph = torch.cuda.CUDAGraph()
        step(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step(0)
        run = graph.replay
    else:
        run = work
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ts = []
    for i in range(n_steps):
        step(i)   # host-side input rotation only: the device work is the graph
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    del flush
    ts = np.array(ts)
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def run_layer(args, log):
    """One decoder layer at batch 1 with the sets predicted inline (predictor, top-k, sparse
    layer), a fresh x for every step: the OPT-6.7B-shaped layer (d 4096, FFN 16384, 32 x 128
    heads, KV 2048, rank 512, 5 % of the neurons = 820, 7 heads, fp16) or, with --shape
    opt125m, the OPT-125m-shaped fp32 layer (d 768, FFN 3072, 12 x 64, KV 128, rank 128, 307
    neurons, 3 heads). Per-step HIP events around graph replays with a 1 GiB write between
    steps (nothing stays in the 256 MB Infinity Cache); the warm number replays back to back
    without the write. Beside it: the dense layer through the same library and through torch,
    and the fp64 oracle on the host on all cores and on one core."""
    import numpy as np
    import torch
    import contextual_activation_sparsity_amd as dv
    from contextual_activation_sparsity_amd import traffic
    import synth
    import synth.device as sdev
    w = {"opt6.7b": synth.OPT6P7B_LAYER, "opt125m": synth.OPT125M_LAYER}[args.shape]
    wb = 2 if w.dtype == "f16" else 4
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t = sdev.layer_on_device(w, 0)
    lw = dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")})
    pw = dv.PredictorWeights(**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")})
    kc = sdev.kv_on_device(w, "k_cache", 0)
    vc = sdev.kv_on_device(w, "v_cache", 0)
    steps = args.layer_steps
    xs = torch.empty(steps, 1, w.d_model, device="cuda")
    for i in range(steps):
        sdev.fill_(xs[i], w.key("x", 0, i), w.x_sigma)
    x = torch.empty(1, w.d_model, device="cuda")
    y = torch.empty_like(x)
    ws = dv.workspace(dims, 1, w.k, w.kh)

    def step(i):
        if torch.cuda.is_current_stream_capturing():
            dv.dv_layer_step(dims, lw, pw, x, x, w.k, w.kh, None, None, kc, vc, w.t_past, y, ws=ws)
        else:
            x.copy_(xs[i % steps])

    med, p10, p90 = timed_single_layer(step, steps, log)
    warm = timed_warm(step, steps)
    tb = traffic.step_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.t_past, w.k, w.kh, wb)
    gbps = tb["total"] / (med * 1e-6) / 1e9
    log(f"[bench] layer {w.name}: median {med:.2f} us (p10 {p10:.2f}, p90 {p90:.2f}), warm {warm:.2f} us, "
        f"{gbps:.0f} GB/s")
    # dense comparators, flushed like the sparse step
    idx = torch.arange(w.d_ffn, dtype=torch.int32, device="cuda")[None].contiguous()
    heads = torch.arange(w.n_heads, dtype=torch.int32, device="cuda")[None].contiguous()
    wsd = dv.workspace(dims, 1, w.d_ffn, w.n_heads)

    def dstep(i):
        if torch.cuda.is_current_stream_capturing():
            dv.dv_layer_step(dims, lw, None, x, None, w.d_ffn, w.n_heads, idx, heads, kc, vc, w.t_past, y, ws=wsd)
        else:
            x.copy_(xs[i % steps])

    n_dense = max(20, steps // 10)
    dmed, _, _ = timed_single_layer(dstep, n_dense, log)
    tfn = torch_dense_layer(w, lw, kc, vc, 1)

    def tstep(i):
        if torch.cuda.is_current_stream_capturing():
            y.copy_(tfn(x))
        else:
            x.copy_(xs[i % steps])

    # hipBLASLt refuses stream capture on this image, so torch's layer is timed eagerly
    tmed, _, _ = timed_single_layer(tstep, n_dense, log, work=lambda: y.copy_(tfn(x)))
    tmode = "eager"
    dbytes = traffic.dense_layer_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.t_past, wb)
    out = {"metric": f"us per sparse decode layer-token (predictor + top-k + layer), {w.name} shape",
           "value": round(med, 3), "unit": "us/layer-token", "n_gpus": 1, "steps": steps, "higher_is_better": False,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: d {w.d_model}, FFN {w.d_ffn}, {w.n_heads} x {w.head_dim} heads, "
                                  f"KV {w.t_past}, rank {w.rank}, k {w.k}, kh {w.kh}, batch 1, inline prediction, "
                                  "fresh x per step",
                      "storage": f"{w.dtype} weights and KV, fp32 activations and accumulation",
                      "timing": "median of per-step HIP events over graph replays, 1 GiB write between steps"},
           "us_p10": round(p10, 3), "us_p90": round(p90, 3),
           "warm_us": round(warm, 3),
           "warm_note": "mean of back-to-back graph replays without the cache flush (weights may stay in the "
                        "256 MB Infinity Cache)",
           "bytes_per_layer_token": int(tb["total"]), "bytes_breakdown": {k: int(v) for k, v in tb.items()},
           "achieved_GBps": round(gbps, 1), "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                        "kernel": "whole step (algorithmic bytes of every kernel / step time)"},
           "dense": {"library_all_selected_us": round(dmed, 2), "torch_dense_layer_us": round(tmed, 2),
                     "bytes": int(dbytes),
                     "torch_launch": tmode,
                     "note": "same flushed timing; torch: F.linear (hipBLASLt) projections + bmm attention"},
           "speedup_vs_dense": round(min(dmed, tmed) / med, 3)}
    del tfn, wsd, t, kc, vc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_layer(w, log)
    return out


def timed_warm(step, n_steps):
    """Mean time of back-to-back graph replays of `step` (no flush between them), in us."""
    import torch
    graph = torch.cuda.CUDAGraph()
    step(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(0)
    for i in range(3):
        step(i)
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_steps):
        step(i)
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n_steps


def cpu_baseline_layer(w, log):
    """The fp64 oracle on layer-tokens of a single-layer workload (predictor, top-k,
    dense-with-mask layer), on every host core and then on one core (BLAS threads limited)."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    t = synth.layer_tensors(w, 0)
    kc = synth.kv_cache(w, "k_cache", 0)
    vc = synth.kv_cache(w, "v_cache", 0)

    def one(step):
        x = synth.x_input(w, step=step)
        c0 = time.perf_counter()
        s_m, s_h = oracle.predict(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"], x)
        S = oracle.topk(s_m.astype(np.float32), w.k)
        Sh = oracle.topk(s_h.astype(np.float32), w.kh)
        oracle.layer(x, t, kc, vc, w.t_past, S, Sh)
        return time.perf_counter() - c0

    res = {}
    for label, limit in (("all_cores", None), ("one_core", 1)):
        ctx = threadpool_limits(limits=limit) if limit else None
        try:
            if ctx is not None:
                ctx.__enter__()
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            secs = []
            while sum(secs) < 10.0 and len(secs) < 200:
                secs.append(one(len(secs)))
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        res[label] = {"value": round(float(np.median(secs)) * 1e6, 1), "unit": "us/layer-token", "cores": int(cores),
                      "reps": len(secs)}
        log(f"[bench] oracle {w.name} {label}: {res[label]}")
    a = res["all_cores"]
    return {"value": a["value"], "unit": "us/layer-token", "cores": a["cores"], "kind": "oracle",
            "sample": f"{a['reps']} {w.name} layer-tokens (fresh x each, median reported): fp64 predictor + top-k + "
                      f"dense-with-mask layer over all {w.d_ffn} neurons and {w.n_heads} heads, KV {w.t_past}",
            "one_core": res["one_core"]}


def run_batched(args, log):
    """One OPT-175B-shaped layer (KV 1024 per sequence) at batch 1..32. Each row's sets are
    the top-k of Zipf(1.1)-skewed popularity scores (Gumbel-top-k: weighted sampling without
    replacement); the step is the batched predictor, the top-k of those scores and the
    layer on the rows' sets (union of the rows' selections on the matrix cores for B >= 2).
    The dense comparator is the same library with every neuron and head selected."""
    import numpy as np
    import torch
    import contextual_activation_sparsity_amd as dv
    from contextual_activation_sparsity_amd import traffic
    import synth
    import synth.device as sdev
    w = synth.OPT175B_BATCHED
    Bmax = 32
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t = sdev.layer_on_device(w, 0)
    lw = dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")})
    pw = dv.PredictorWeights(**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")})
    wb = w.with_(batch=Bmax)
    kc = sdev.kv_on_device(wb, "k_cache", 0)
    vc = sdev.kv_on_device(wb, "v_cache", 0)
    steps = max(5, min(args.steps, 30))
    points = []
    sizes = [int(v) for v in args.batch_sizes.split(",") if v.strip()]
    if not sizes or any(not 1 <= B <= Bmax for B in sizes):
        raise SystemExit(f"--batch-sizes must list values in 1..{Bmax}")
    for B in sizes:
        wB = w.with_(batch=B)
        zs_m = torch.from_numpy(synth.zipf_scores(wB, w.d_ffn, "sel_mlp")).cuda()
        zs_h = torch.from_numpy(synth.zipf_scores(wB, w.n_heads, "sel_head")).cuda()
        idx = torch.empty(B, w.k, dtype=torch.int32, device="cuda")
        heads = torch.empty(B, w.kh, dtype=torch.int32, device="cuda")
        dv.dv_topk(zs_m, w.k, idx)
        dv.dv_topk(zs_h, w.kh, heads)
        torch.cuda.synchronize()
        nU = int(np.unique(idx.cpu().numpy()).size)
        nUh = int(np.unique(heads.cpu().numpy()).size)
        xs = torch.empty(steps, B, w.d_model, device="cuda")
        for i in range(steps):
            sdev.fill_(xs[i], w.key("x", 0, i), w.x_sigma)
        x = torch.empty(B, w.d_model, device="cuda")
        y = torch.empty_like(x)
        s_m = torch.empty(B, w.d_ffn, device="cuda")
        s_h = torch.empty(B, w.n_heads, device="cuda")
        ws = dv.workspace(dims, B, w.k, w.kh)
        tws_m = torch.empty(dv.dv_topk_workspace_bytes(B, w.d_ffn), dtype=torch.uint8, device="cuda")
        tws_h = torch.empty(dv.dv_topk_workspace_bytes(B, w.n_heads), dtype=torch.uint8, device="cuda")
        kB, vB = kc[:B], vc[:B]

        def step(i):
            if torch.cuda.is_current_stream_capturing():
                dv.dv_predict(dims, pw, x, s_m, s_h, ws)
                dv.dv_topk(zs_m, w.k, idx, tws_m)
                dv.dv_topk(zs_h, w.kh, heads, tws_h)
                dv.dv_layer_step(dims, lw, None, x, None, w.k, w.kh, idx, heads, kB, vB, w.t_past, y, ws=ws)
            else:
                x.copy_(xs[i % steps])

        med, p10, p90 = timed_single_layer(step, steps, log)
        tb = traffic.step_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.t_past, nU, nUh, 2, batch=B,
                                kh_rows_kv=B * w.kh)
        # dense comparator: every neuron and head for every row, same library
        ai = torch.arange(w.d_ffn, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
        ah = torch.arange(w.n_heads, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
        wsd = dv.workspace(dims, B, w.d_ffn, w.n_heads)

        def dstep(i):
            if torch.cuda.is_current_stream_capturing():
                dv.dv_layer_step(dims, lw, None, x, None, w.d_ffn, w.n_heads, ai, ah, kB, vB, w.t_past, y, ws=wsd)
            else:
                x.copy_(xs[i % steps])

        dmed, _, _ = timed_single_layer(dstep, max(3, steps // 3), log)
        del wsd, ai, ah
        # dense comparator in torch: hipBLASLt F.linear over the B rows, bmm attention
        tfn = torch_dense_layer(w, lw, kc, vc, B)

        def tstep(i):
            if torch.cuda.is_current_stream_capturing():
                y.copy_(tfn(x))
            else:
                x.copy_(xs[i % steps])

        # hipBLASLt refuses stream capture on this image, so torch's layer is timed eagerly
        tmed, _, _ = timed_single_layer(tstep, max(3, steps // 3), log, work=lambda: y.copy_(tfn(x)))
        del tfn
        pt = {"batch": B, "union_neurons": nU, "union_heads": nUh, "us_per_step": round(med, 2),
              "us_p10": round(p10, 2), "us_p90": round(p90, 2), "us_per_token": round(med / B, 2),
              "bytes_per_step": int(tb["total"]), "achieved_GBps": round(tb["total"] / (med * 1e-6) / 1e9, 1),
              "dense_us_per_step": round(dmed, 2), "speedup_vs_dense": round(dmed / med, 3),
              "torch_dense_us_per_step": round(tmed, 2), "speedup_vs_torch_dense": round(tmed / med, 3),
              "speedup_vs_faster_dense": round(min(dmed, tmed) / med, 3)}
        log(f"[bench] batched B={B}: {pt}")
        points.append(pt)
        del ws, xs
        torch.cuda.empty_cache()
    return {"metric": "us per batched sparse decode step (predictor + top-k + layer), OPT-175B shape",
            "value": points[-1]["us_per_step"], "unit": "us/step", "n_gpus": 1, "steps": steps,
            "higher_is_better": False, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "opt175b-shaped layer, batch 1..32, Zipf(1.1) selections, KV 1024",
                       "k": w.k, "kh": w.kh, "rank": w.rank,
                       "dense": "dense_us_per_step: this library with every neuron and head selected; "
                                "torch_dense_us_per_step: torch F.linear (hipBLASLt) + bmm attention, same flushed "
                                "timing but eager launches (hipBLASLt refuses stream capture)",
                       "timing": "median of per-step HIP events over graph replays, 1 GiB write between steps"},
            "points": points}


def run_sweep(args, log):
    """OPT-66B-shaped layer (KV 2048, rank 1000) at batch 1 over MLP densities x head
    densities: the full step with inline prediction (predictor, top-k, sparse layer), fresh
    x per step, against the dense layer through the same library."""
    import torch
    import contextual_activation_sparsity_amd as dv
    from contextual_activation_sparsity_amd import traffic
    import synth
    import synth.device as sdev
    import numpy as np
    w = synth.OPT66B_LAYER
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t = sdev.layer_on_device(w, 0)
    lw = dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")})
    pw = dv.PredictorWeights(**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")})
    kc = sdev.kv_on_device(w, "k_cache", 0)
    vc = sdev.kv_on_device(w, "v_cache", 0)
    steps = max(5, min(args.steps, 30))
    xs = torch.empty(steps, 1, w.d_model, device="cuda")
    for i in range(steps):
        sdev.fill_(xs[i], w.key("x", 0, i), w.x_sigma)
    x = torch.empty(1, w.d_model, device="cuda")
    y = torch.empty_like(x)
    points = []
    cells = [(dm, dhd) for dm in synth.SWEEP_MLP for dhd in synth.SWEEP_HEAD]
    if args.sweep_cells:
        want = [tuple(float(v) for v in c.split(":")) for c in args.sweep_cells.split(",") if c.strip()]
        cells = [c for c in cells if any(abs(c[0] - a) < 1e-9 and abs(c[1] - b) < 1e-9 for a, b in want)]
        if len(cells) != len(want):
            raise SystemExit(f"--sweep-cells must name cells of {synth.SWEEP_MLP} x {synth.SWEEP_HEAD}")
    for dm, dhd in cells:
        k, kh = synth.count_at(dm, w.d_ffn), synth.count_at(dhd, w.n_heads)
        ws = dv.workspace(dims, 1, k, kh)

        def step(i):
            if torch.cuda.is_current_stream_capturing():
                dv.dv_layer_step(dims, lw, pw, x, x, k, kh, None, None, kc, vc, w.t_past, y, ws=ws)
            else:
                x.copy_(xs[i % steps])

        med, p10, p90 = timed_single_layer(step, steps, log)
        tb = traffic.step_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.t_past, k, kh, 2)
        pt = {"mlp_density": dm, "head_density": dhd, "k": k, "kh": kh, "us": round(med, 2),
              "us_p10": round(p10, 2), "us_p90": round(p90, 2), "bytes": int(tb["total"]),
              "achieved_GBps": round(tb["total"] / (med * 1e-6) / 1e9, 1)}
        log(f"[bench] sweep {pt}")
        points.append(pt)
    idx = torch.arange(w.d_ffn, dtype=torch.int32, device="cuda")[None].contiguous()
    heads = torch.arange(w.n_heads, dtype=torch.int32, device="cuda")[None].contiguous()
    wsd = dv.workspace(dims, 1, w.d_ffn, w.n_heads)

    def dstep(i):
        if torch.cuda.is_current_stream_capturing():
            dv.dv_layer_step(dims, lw, None, x, None, w.d_ffn, w.n_heads, idx, heads, kc, vc, w.t_past, y, ws=wsd)
        else:
            x.copy_(xs[i % steps])

    dmed, _, _ = timed_single_layer(dstep, steps, log)
    dbytes = traffic.dense_layer_bytes(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.t_past, 2)
    del wsd
    # The same cells in lookahead mode, as the method runs them: a stack of L independent
    # layers of this shape, the sets of layer l+1 predicted from the input of layer l on a side
    # stream while layer l runs (layer 0's prediction is the only serial one). Timed over graph
    # replays of the whole stack (L layers move far more than the Infinity Cache holds), fresh x
    # copied in before each replay; us per layer-token = step / L.
    L = max(2, args.sweep_layers)
    layers, preds, kcs, vcs = [lw], [pw], [kc], [vc]
    for l in range(1, L):
        tl = sdev.layer_on_device(w, l)
        layers.append(dv.LayerWeights(**{k: tl[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1",
                                                              "w2", "b2")}))
        preds.append(dv.PredictorWeights(**{k: tl[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")}))
        kcs.append(sdev.kv_on_device(w, "k_cache", l))
        vcs.append(sdev.kv_on_device(w, "v_cache", l))
    side = torch.cuda.Stream()
    for pt in points:
        k, kh = pt["k"], pt["kh"]
        sws = dv.stack_workspace(dims, 1, k, kh)
        dv.dv_lookahead_stack(dims, layers, preds, x, k, kh, kcs, vcs, w.t_past, y, ws=sws, side_stream=side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dv.dv_lookahead_stack(dims, layers, preds, x, k, kh, kcs, vcs, w.t_past, y, ws=sws, side_stream=side)
        ts = []
        for i in range(steps + 2):
            x.copy_(xs[i % steps])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3 / L)
        us = float(np.median(ts))
        pt["lookahead_us"] = round(us, 2)
        pt["lookahead_GBps"] = round(pt["bytes"] / (us * 1e-6) / 1e9, 1)
        log(f"[bench] sweep lookahead mlp {pt['mlp_density']} head {pt['head_density']}: {us:.2f} us/layer-token")
        del g, sws
    del layers, preds, kcs, vcs
    torch.cuda.empty_cache()
    at5 = next((p for p in points if p["mlp_density"] == 0.05 and p["head_density"] == 0.20), points[0])
    return {"metric": "us per sparse decode layer-token over MLP x head density, OPT-66B shape",
            "value": at5["us"], "unit": "us/layer-token", "n_gpus": 1, "steps": steps, "higher_is_better": False,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "opt66b-shaped layer density sweep, batch 1, inline prediction, KV 2048",
                       "timing": "us: serial step (predictor, top-k, layer), median of per-step HIP events over "
                                 "graph replays, 1 GiB write between steps; lookahead_us: the same cell in a stack "
                                 f"of {L} layers with the next layer's prediction on a side stream, median "
                                 "replay time / layers"},
            "dense": {"us": round(dmed, 2), "bytes": int(dbytes),
                      "achieved_GBps": round(dbytes / (dmed * 1e-6) / 1e9, 1)},
            "points": points}


def run_blocked(args, log):
    """OPT-175B-shaped MLP at 5 % density: selection + sparse MLP with single neurons
    (top-k of the scores) against whole blocks of 32 or 64 neurons (top-k of the block
    maxima), batch 1, per-step HIP events with a 1 GiB write between steps. The scores are
    synthetic (seeded normal), so the overlap of the two selections says nothing about a
    trained model; it is reported to show what blocking costs in selection on such scores."""
    import numpy as np
    import torch
    import contextual_activation_sparsity_amd as dv
    import synth
    import synth.device as sdev
    w = synth.OPT175B_BATCHED
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t = sdev.layer_on_device(w, 0)
    lw = dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")})
    steps = max(5, min(args.steps, 30))
    F, d = w.d_ffn, w.d_model
    sc = torch.empty(steps, 1, F, device="cuda")
    xs = torch.empty(steps, 1, d, device="cuda")
    for i in range(steps):
        sdev.fill_(sc[i], w.key("scores", 0, i), 1.0)
        sdev.fill_(xs[i], w.key("x", 0, i), 1.0)
    s_in = torch.empty(1, F, device="cuda")
    x = torch.empty(1, d, device="cuda")
    y = torch.empty_like(x)
    points = []
    for bs in (1, 32, 64):
        kb = max(1, int(round(w.k / bs)))
        nb = F // bs
        sel = torch.empty(1, kb, dtype=torch.int32, device="cuda")
        bsc = torch.empty(1, nb, device="cuda")
        ws = dv.workspace(dims, 1, kb * bs, 0)
        tws = torch.empty(dv.dv_topk_workspace_bytes(1, nb), dtype=torch.uint8, device="cuda")

        def step(i):
            if torch.cuda.is_current_stream_capturing():
                if bs == 1:
                    dv.dv_topk(s_in, kb, sel, tws)
                    dv.dv_sparse_mlp(dims, lw, x, sel, kb, y, ws)
                else:
                    dv.dv_block_scores(s_in, bs, bsc)
                    dv.dv_topk(bsc, kb, sel, tws)
                    dv.dv_sparse_mlp_blocked(dims, lw, x, sel, kb, bs, y, ws)
            else:
                s_in.copy_(sc[i % steps])
                x.copy_(xs[i % steps])

        med, p10, p90 = timed_single_layer(step, steps, log)
        # overlap with the per-neuron top-k on the same scores (last step's inputs)
        s_host = s_in.cpu().numpy()[0]
        top = set(np.argsort(-s_host, kind="stable")[:w.k].tolist())
        if bs == 1:
            kept = 1.0
        else:
            chosen = sel.cpu().numpy()[0]
            neurons = set((chosen[:, None] * bs + np.arange(bs)[None]).ravel().tolist())
            kept = len(top & neurons) / len(top)
        mb = 2 * kb * bs * d * 2 / 1e6
        pt = {"block": bs, "blocks_kept": kb, "neurons_kept": kb * bs, "us": round(med, 2), "us_p10": round(p10, 2),
              "us_p90": round(p90, 2), "mlp_weight_MB": round(mb, 1),
              "achieved_GBps_weights": round(mb * 1e6 / (med * 1e-6) / 1e9, 1),
              "share_of_neuron_topk_kept": round(kept, 4)}
        log(f"[bench] blocked {pt}")
        points.append(pt)
    return {"metric": "us per selection + sparse MLP step, single neurons vs 32/64-neuron blocks, OPT-175B shape",
            "value": points[0]["us"], "unit": "us/step", "n_gpus": 1, "steps": steps, "higher_is_better": False,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "opt175b-shaped MLP, batch 1, 5 % of neurons, synthetic scores",
                       "timing": "median of per-step HIP events over graph replays, 1 GiB write between steps"},
            "points": points}


def run_decode(args, log):
    """Consecutive decode tokens through the 24-layer OPT-175B-shaped stack with the KV
    growing by one slot per token: one call of the stack with per-row lengths on the device
    is captured once in a HIP graph and replayed per token (the lengths advance on the
    device, fresh x is copied in before each replay). B = 1 from KV 2048, and B = 8 with
    the rows spread over KV 256..2048 (union path). Beside it: the fixed-length stack step
    (graph replay at KV 2048, the same step every time)."""
    import numpy as np
    import torch
    import contextual_activation_sparsity_amd as dv
    import synth
    import synth.device as sdev
    w = synth.OPT175B_STACK
    L = w.n_layers
    n_tok = max(8, min(args.steps, 64))
    warm = 4
    t_max = w.t_past + n_tok + warm + 1
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, t_max, w.dtype)
    layers, preds = [], []
    for l in range(L):
        t = sdev.layer_on_device(w, l)
        layers.append(dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1",
                                                             "w2", "b2")}))
        preds.append(dv.PredictorWeights(**{k: t[k] for k in ("p1_mlp", "p2_mlp", "p1_head", "p2_head")}))
    side = torch.cuda.Stream()
    lines = []
    for B, lengths in ((1, [w.t_past]), (8, [int(v) for v in np.linspace(256, w.t_past, 8)])):
        kcs, vcs = [], []
        for l in range(L):
            for which, lst in (("k_cache", kcs), ("v_cache", vcs)):
                c = torch.empty(B, w.n_heads, t_max, w.head_dim, dtype=torch.float16, device="cuda")
                sdev.fill_(c, w.key(which, l), w.kv_sigma)
                lst.append(c)

        def reset():
            for c in kcs + vcs:
                for b, T in enumerate(lengths):
                    c[b, :, T:].zero_()
            t_rows.copy_(torch.tensor(lengths, dtype=torch.int32))

        t_rows = torch.empty(B, dtype=torch.int32, device="cuda")
        xs = torch.empty(n_tok + warm, B, w.d_model, device="cuda")
        for i in range(n_tok + warm):
            sdev.fill_(xs[i], w.key("x", 0, 1000 + i), w.x_sigma)
        x_in = torch.empty(B, w.d_model, device="cuda")
        y = torch.empty_like(x_in)
        ws = dv.stack_workspace(dims, B, w.k, w.kh)
        reset()
        x_in.copy_(xs[0])
        # per-device set-up outside the capture, on scratch copies of the state
        dv.dv_decode_step(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, t_rows.clone(), y, advance=False, ws=ws,
                          side_stream=side)
        torch.cuda.synchronize()
        reset()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dv.dv_decode_step(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, t_rows, y, advance=True, ws=ws,
                              side_stream=side)
        torch.cuda.synchronize()
        for i in range(warm):
            x_in.copy_(xs[i])
            graph.replay()
        torch.cuda.synchronize()
        ts = []
        for i in range(n_tok):
            x_in.copy_(xs[warm + i])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        t_end = t_rows.cpu().numpy()
        assert np.array_equal(t_end, np.array(lengths) + warm + n_tok), t_end
        ts = np.array(ts)
        line = {"batch": B, "kv_start": lengths, "tokens": n_tok, "us_per_token_median": round(float(np.median(ts)), 2),
                "us_first": round(float(ts[0]), 2), "us_last": round(float(ts[-1]), 2),
                "us_per_layer_token": round(float(np.median(ts)) / L / B, 3),
                "tokens_per_s": round(B * 1e6 / float(np.median(ts)), 1)}
        # the same shape at a fixed length: the stack step replayed at one position
        if B == 1:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                dv.dv_lookahead_stack(dims, layers, preds, x_in, w.k, w.kh, kcs, vcs, w.t_past, y, ws=ws,
                                      side_stream=side)
            torch.cuda.synchronize()
            for _ in range(3):
                g2.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(n_tok):
                g2.replay()
            e1.record()
            torch.cuda.synchronize()
            line["fixed_kv_us_per_token"] = round(e0.elapsed_time(e1) * 1e3 / n_tok, 2)
            del g2
        log(f"[bench] decode {line}")
        lines.append(line)
        del graph, kcs, vcs, ws, xs
        torch.cuda.empty_cache()
    return {"metric": "us per decode token through the 24-layer OPT-175B-shaped stack, KV growing per token",
            "value": lines[0]["us_per_token_median"], "unit": "us/token", "n_gpus": 1, "steps": n_tok,
            "higher_is_better": False, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "opt175b-shaped 24-layer stack, consecutive tokens, per-row KV lengths on the "
                                   "device advanced by the step, one graph replayed per token",
                       "k": w.k, "kh": w.kh, "rank": w.rank,
                       "timing": "HIP events around each replay; fresh x copied in before it"},
            "lines": lines}


def run_train(args, log):
    """Predictor training for the OPT-125m-shaped layer (fp32): dense-layer targets for 8192
    training and 1024 held-out inputs (inputs near a 32-dimensional affine subspace), then
    300 full-batch momentum steps for the neuron predictor (lr 3) and the head predictor
    (lr 0.3), then recall@k of the library's predictor + top-k on the held-out inputs. The
    targets and every step run on the GPU; recall is counted on the host."""
    import numpy as np
    import torch
    import contextual_activation_sparsity_amd as dv
    import synth
    w = synth.OPT125M_TRAIN
    M, Mh, steps = 8192, 1024, 300
    dims = dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in synth.layer_tensors(w).items()}
    lw = dv.LayerWeights(**{k: t[k] for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")})

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def targets(n, split):
        x = torch.from_numpy(synth.lowdim_x(w, n, split=split)).cuda()
        wc = w.with_(batch=n)
        kc = torch.zeros(synth.kv_shape(wc), dtype=torch.float32, device="cuda")   # no past tokens
        vc = torch.zeros_like(kc)
        fire = torch.empty(n, w.d_ffn, dtype=torch.uint8, device="cuda")
        hn = torch.empty(n, w.n_heads, device="cuda")
        ws = dv.workspace(dims, n, w.d_ffn, w.n_heads)
        dv.dv_layer_labels(dims, lw, x, kc, vc, w.t_past, fire=fire, head_norm=hn, ws=ws)   # warm
        e0, e1 = ev(), ev()
        e0.record()
        dv.dv_layer_labels(dims, lw, x, kc, vc, w.t_past, fire=fire, head_norm=hn, ws=ws)
        top = torch.empty(n, w.kh, dtype=torch.int32, device="cuda")
        dv.dv_topk(hn, w.kh, top)
        e1.record()
        torch.cuda.synchronize()
        hl = torch.zeros(n, w.n_heads, dtype=torch.uint8, device="cuda")
        hl.scatter_(1, top.long(), 1)
        return x, fire, hl, e0.elapsed_time(e1) * 1e3

    x, fire, hlab, us_lab = targets(M, 0)
    xh, fire_h, hlab_h, _ = targets(Mh, 1)
    log(f"[bench] targets for {M} inputs: {us_lab:.0f} us; firing share {fire.float().mean().item():.4f}")

    def recall(sets, lab):
        sets, lab = sets.cpu().numpy(), lab.cpu().numpy()
        pos = lab.sum(1)
        hit = np.take_along_axis(lab, sets.astype(np.int64), 1).sum(1)
        return float(np.mean(np.where(pos > 0, hit / np.maximum(pos, 1), 1.0)))

    def select(p1m, p2m, p1h, p2h):
        pw = dv.PredictorWeights(p1_mlp=p1m, p2_mlp=p2m, p1_head=p1h, p2_head=p2h)
        s_m = torch.empty(Mh, w.d_ffn, device="cuda")
        s_h = torch.empty(Mh, w.n_heads, device="cuda")
        dv.dv_predict(dims, pw, xh, s_m, s_h, dv.workspace(dims, Mh, w.k, w.kh))
        S = torch.empty(Mh, w.k, dtype=torch.int32, device="cuda")
        Sh = torch.empty(Mh, w.kh, dtype=torch.int32, device="cuda")
        dv.dv_topk(s_m, w.k, S)
        dv.dv_topk(s_h, w.kh, Sh)
        torch.cuda.synchronize()
        return recall(S, fire_h), recall(Sh, hlab_h)

    start = select(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"])

    def prior(lab_train, lab_test, k):
        freq = lab_train.float().mean(0).cpu().numpy()
        top = np.sort(np.argsort(-freq, kind="stable")[:k])
        return recall(torch.from_numpy(np.tile(top, (Mh, 1))), lab_test)

    def train(p1, p2, y, lr):
        p1, p2 = p1.clone(), p2.clone()
        v1, v2 = torch.zeros_like(p1), torch.zeros_like(p2)
        loss = torch.zeros(steps, device="cuda")
        N, r = p2.shape
        ws = torch.empty(dv.dv_predictor_train_workspace_bytes(M, w.d_model, N, r), dtype=torch.uint8, device="cuda")
        dv.dv_predictor_train_step(x, y, p1.clone(), p2.clone(), v1.clone(), v2.clone(), lr, 0.9, loss[:1], ws)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(steps):
            dv.dv_predictor_train_step(x, y, p1, p2, v1, v2, lr, 0.9, loss[i:i + 1], ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        flop = 2.0 * M * (2 * r * w.d_model + 3 * r * N)
        lv = loss.cpu().numpy()
        return p1, p2, {"us_per_step": round(us, 1), "gflop_per_step": round(flop / 1e9, 3),
                        "tflops": round(flop / (us * 1e-6) / 1e12, 2), "loss_first": round(float(lv[0]), 5),
                        "loss_last": round(float(lv[-1]), 5)}

    p1m, p2m, tm = train(t["p1_mlp"], t["p2_mlp"], fire, 3.0)
    p1h, p2h, th = train(t["p1_head"], t["p2_head"], hlab, 0.3)
    end = select(p1m, p2m, p1h, p2h)
    res = {"neurons": {"k": w.k, "recall_start": round(start[0], 4), "recall_trained": round(end[0], 4),
                       "recall_most_frequent": round(prior(fire, fire_h, w.k), 4), **tm},
           "heads": {"kh": w.kh, "recall_start": round(start[1], 4), "recall_trained": round(end[1], 4),
                     "recall_most_frequent": round(prior(hlab, hlab_h, w.kh), 4), **th}}
    log(f"[bench] train {res}")
    return {"metric": "recall@k of the trained rank-128 predictors on held-out inputs; train-step time",
            "value": res["neurons"]["recall_trained"], "unit": "recall", "n_gpus": 1, "steps": steps,
            "higher_is_better": True, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "opt125m-shaped layer fp32, 8192 training / 1024 held-out inputs near a "
                                   "32-dimensional affine subspace, biases shifted so ~10 % of neurons fire",
                       "rank": w.rank, "momentum": 0.9, "targets_us": round(us_lab, 1),
                       "fp32_peak_tflops": 157.3},
            "results": res}


def cpu_baseline(w, log):
    """The fp64 oracle, as it stands, on layer-tokens of the same shape: predictor over
    all neurons and heads, exact top-k, then the dense-with-mask layer (every neuron's and
    head's projection computed, masks applied). Weights drawn on the host (not timed)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.time()
    t = synth.layer_tensors(w, 0)
    kc = synth.kv_cache(w, "k_cache", 0)
    vc = synth.kv_cache(w, "v_cache", 0)
    log(f"[bench] oracle inputs drawn on the host in {time.time() - t0:.1f}s")
    # Repeat whole layer-tokens (fresh x each) until about 10 s of CPU work has been timed.
    secs = []
    while sum(secs) < 10.0 and len(secs) < 8:
        x = synth.x_input(w, step=len(secs))
        c0 = time.perf_counter()
        s_m, s_h = oracle.predict(t["p1_mlp"], t["p2_mlp"], t["p1_head"], t["p2_head"], x)
        S = oracle.topk(s_m.astype(np.float32), w.k)
        Sh = oracle.topk(s_h.astype(np.float32), w.kh)
        oracle.layer(x, t, kc, vc, w.t_past, S, Sh)
        secs.append(time.perf_counter() - c0)
    sec = float(np.median(secs))
    log(f"[bench] oracle: {len(secs)} layer-tokens, median {sec:.2f}s each on {cores} threads")
    return {"value": round(sec * 1e6, 1), "unit": "us/layer-token", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(secs)} OPT-175B-shaped layer-tokens of layer 0 (steps 0..{len(secs) - 1}, median "
                      "reported): fp64 predictor + top-k + dense-with-mask layer over all 49152 neurons and "
                      "96 heads, KV 2048"}


if __name__ == "__main__":
    sys.exit(main())
