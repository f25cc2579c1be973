"""Predictor training on the GPU (dense-layer targets, full-batch steps, recall through the
library's own predictor and top-k) against the fp64 oracle on the same seeded inputs.

Bars: targets' pre-activations and head norms within the single-layer bar of their dtype; a
target bit may differ only where the oracle's pre-activation is within 1e-4 * RMS of zero
(fp32 decides it there), and a head target only where the kh-th and (kh+1)-th norms are that
close. Training: each step's loss within 1e-5 relative, and the parameters' total change
within 1e-3 of the oracle's change (fp32 GEMMs against fp64; the errors stay proportional
because the update is linear in the gradients)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import W_RAG16, W_RAG32, assert_close, kv_host, layer_weights, rms, to_dev

import contextual_activation_sparsity_amd as dvmod

pytestmark = pytest.mark.gpu


def dims_of(w):
    return dvmod.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)


def gpu_train(dv, x, y, p1, p2, steps, lr, mu):
    xd, yd = torch.from_numpy(np.ascontiguousarray(x)).cuda(), torch.from_numpy(np.ascontiguousarray(y)).cuda()
    a = torch.from_numpy(np.ascontiguousarray(p1, np.float32)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(p2, np.float32)).cuda()
    v1, v2 = torch.zeros_like(a), torch.zeros_like(b)
    loss = torch.zeros(max(steps, 1), device="cuda")
    ws = torch.empty(dv.dv_predictor_train_workspace_bytes(x.shape[0], x.shape[1], y.shape[1], p1.shape[0]),
                     dtype=torch.uint8, device="cuda")
    for s in range(steps):
        dv.dv_predictor_train_step(xd, yd, a, b, v1, v2, lr, mu, loss[s:s + 1], ws)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy(), loss.cpu().numpy()[:steps]


def check_train(dv, x, y, p1, p2, steps, lr, mu, what):
    a, b, lg = gpu_train(dv, x, y, p1, p2, steps, lr, mu)
    ra, rb, lo = oracle.train_predictor(x, y, p1, p2, steps, lr, mu)
    assert np.allclose(lg, lo, rtol=1e-5, atol=0), f"{what}: losses {lg} vs {lo}"
    for got, ref, init, name in ((a, ra, p1, "p1"), (b, rb, p2, "p2")):
        dg = got.astype(np.float64) - init.astype(np.float64)
        dr = ref - init.astype(np.float64)
        err = np.max(np.abs(dg - dr))
        assert err <= 1e-3 * np.max(np.abs(dr)), f"{what} {name}: change off by {err:.3e} of {np.max(np.abs(dr)):.3e}"


@pytest.mark.parametrize("shape", [(200, 100, 70, 20), (64, 768, 12, 128), (512, 768, 3072, 128)],
                         ids=["ragged", "opt125m-heads", "opt125m-neurons"])
def test_train_steps_match_oracle(dv, shape):
    M, d, N, r = shape
    w = synth.OPT125M_TRAIN.with_(d_model=d)
    x = synth.lowdim_x(w, M)
    y = synth.random_labels(w, M, N, 0.1)
    p1 = synth.tensor(w.key("p1_mlp"), (r, d), 0.05, "f32")
    p2 = synth.tensor(w.key("p2_mlp"), (N, r), 0.05, "f32")
    lr = 0.3 if N < 100 else 3.0
    check_train(dv, x, y, p1, p2, 3, lr, 0.9, f"M={M} d={d} N={N} r={r}")


def test_train_step_is_deterministic(dv):
    w = synth.OPT125M_TRAIN
    x = synth.lowdim_x(w, 300)
    y = synth.random_labels(w, 300, 3072, 0.1)
    p1 = synth.tensor(w.key("p1_mlp"), (128, 768), 0.05, "f32")
    p2 = synth.tensor(w.key("p2_mlp"), (3072, 128), 0.05, "f32")
    r1 = gpu_train(dv, x, y, p1, p2, 2, 3.0, 0.9)
    r2 = gpu_train(dv, x, y, p1, p2, 2, 3.0, 0.9)
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)


def labels_on_gpu(dv, w, t, x, kc, vc):
    B = x.shape[0]
    dims = dims_of(w)
    d = to_dev(t)
    fire = torch.empty(B, w.d_ffn, dtype=torch.uint8, device="cuda")
    pre = torch.empty(B, w.d_ffn, device="cuda")
    hn = torch.empty(B, w.n_heads, device="cuda")
    dv.dv_layer_labels(dims, layer_weights(d), torch.from_numpy(x).cuda(), torch.from_numpy(kc).cuda(),
                       torch.from_numpy(vc).cuda(), w.t_past, fire=fire, preact=pre, head_norm=hn)
    top = torch.empty(B, w.kh, dtype=torch.int32, device="cuda")
    dv.dv_topk(hn, w.kh, top)
    torch.cuda.synchronize()
    return fire.cpu().numpy(), pre.cpu().numpy(), hn.cpu().numpy(), top.cpu().numpy()


@pytest.mark.parametrize("which", ["opt125m-train", "ragged-f32-past", "ragged-f16-past"])
def test_layer_labels_match_oracle(dv, which):
    if which == "opt125m-train":
        w = synth.OPT125M_TRAIN.with_(batch=64)
        x = synth.lowdim_x(w, 64)
    else:
        w = (W_RAG32 if which == "ragged-f32-past" else W_RAG16).with_(batch=5, kh=3)
        x = synth.x_input(w, step=2)
    t = synth.layer_tensors(w)
    kc, vc = kv_host(w, "k_cache"), kv_host(w, "v_cache")
    fire, pre, hn, top = labels_on_gpu(dv, w, t, x, kc, vc)
    ref = oracle.layer_labels(x, t, kc, vc, w.t_past, w.kh)
    assert_close(pre, ref["a"], w.dtype, f"{which} pre-activations")
    assert_close(hn, ref["head_norm"], w.dtype, f"{which} head norms")
    band = 1e-4 * rms(ref["a"])
    clear = np.abs(ref["a"]) > band
    assert np.array_equal(fire[clear], ref["fire"][clear]), f"{which}: target bits differ away from zero"
    assert np.array_equal(fire, (pre > 0).astype(np.uint8))
    for b in range(x.shape[0]):
        srt = np.sort(ref["head_norm"][b])[::-1]
        if w.kh < w.n_heads and srt[w.kh - 1] - srt[w.kh] <= 1e-4 * srt[0]:
            continue
        assert np.array_equal(top[b], ref["head_top"][b]), f"{which} row {b}: head targets differ"


def test_trained_predictor_recall_matches_oracle(dv):
    """Targets on the GPU, training on the GPU, selection through dv_predict + dv_topk on
    held-out inputs: recall within 0.03 of the oracle's pipeline, and far above the start."""
    w = synth.OPT125M_TRAIN
    M, Mh, steps, lr = 1024, 256, 60, 3.0
    t = synth.layer_tensors(w)
    x, xh = synth.lowdim_x(w, M, split=0), synth.lowdim_x(w, Mh, split=1)
    wt, wh = w.with_(batch=M), w.with_(batch=Mh)
    kt, vt = kv_host(wt, "k_cache"), kv_host(wt, "v_cache")
    kh_, vh_ = kv_host(wh, "k_cache"), kv_host(wh, "v_cache")
    fire, *_ = labels_on_gpu(dv, wt, t, x, kt, vt)
    fire_h, *_ = labels_on_gpu(dv, wh, t, xh, kh_, vh_)
    a, b, lg = gpu_train(dv, x, fire, t["p1_mlp"], t["p2_mlp"], steps, lr, 0.9)
    # selection on held-out inputs through the library
    dims = dims_of(wh)
    pw = dvmod.PredictorWeights(p1_mlp=torch.from_numpy(a).cuda(), p2_mlp=torch.from_numpy(b).cuda(),
                                p1_head=torch.from_numpy(t["p1_head"]).cuda(), p2_head=torch.from_numpy(t["p2_head"]).cuda())
    s_m = torch.empty(Mh, w.d_ffn, device="cuda")
    s_h = torch.empty(Mh, w.n_heads, device="cuda")
    dv.dv_predict(dims, pw, torch.from_numpy(xh).cuda(), s_m, s_h, dv.workspace(dims, Mh, w.k, w.kh))
    S = torch.empty(Mh, w.k, dtype=torch.int32, device="cuda")
    dv.dv_topk(s_m, w.k, S)
    torch.cuda.synchronize()
    sel = S.cpu().numpy().astype(np.int64)
    pos = fire_h.sum(1)
    hit = np.take_along_axis(fire_h, sel, 1).sum(1)
    rec_gpu = float(np.mean(np.where(pos > 0, hit / np.maximum(pos, 1), 1.0)))   # counted here, not by the oracle
    # the oracle's own pipeline
    lab = oracle.layer_labels(x, t, kt, vt, 0, w.kh)
    lab_h = oracle.layer_labels(xh, t, kh_, vh_, 0, w.kh)
    ra, rb, lo = oracle.train_predictor(x, lab["fire"], t["p1_mlp"], t["p2_mlp"], steps, lr, 0.9)
    rec_or = float(oracle.recall(oracle.topk(((xh.astype(np.float64) @ ra.T) @ rb.T).astype(np.float32), w.k),
                                 lab_h["fire"]).mean())
    rec_init = float(oracle.recall(oracle.topk(((xh.astype(np.float64) @ t["p1_mlp"].T.astype(np.float64))
                                                @ t["p2_mlp"].T.astype(np.float64)).astype(np.float32), w.k),
                                   lab_h["fire"]).mean())
    print(f"recall@k: start {rec_init:.3f}, oracle {rec_or:.3f}, library {rec_gpu:.3f}; loss {lg[0]:.4f} -> {lg[-1]:.4f}")
    assert abs(rec_gpu - rec_or) <= 0.03
    assert rec_gpu >= 2.0 * rec_init
