"""dv_layer_step_noalloc (GPU): the allocation-free entry point against dv_layer_step with a
workspace, bit for bit, on two calls in a row, the second on a smaller input (so the fixed
scratch array still holds the first call's larger contents): an OPT-6.7B-shaped layer at
B = 4 on the batched union path with sets predicted inline, then a ragged fp16 layer at
B = 1 with given sets. Outputs, exported sets and appended caches must all match."""
import numpy as np
import pytest
import torch

import synth
from helpers import W_C2, W_RAG16, dims_of, kv_host, layer_weights, pred_weights, random_sets, to_dev

pytestmark = pytest.mark.gpu


_LAYERS = {}


def case(dv, w, B, inline, noalloc, seed):
    if w.name not in _LAYERS:
        _LAYERS[w.name] = to_dev(synth.layer_tensors(w))
    t = _LAYERS[w.name]
    wc = w.with_(batch=B)
    x = torch.from_numpy(synth.x_input(wc, step=seed)).cuda()
    kc = torch.from_numpy(kv_host(wc, "k_cache")).cuda()
    vc = torch.from_numpy(kv_host(wc, "v_cache")).cuda()
    out = torch.empty_like(x)
    io = torch.empty(B, w.k, dtype=torch.int32, device="cuda")
    ho = torch.empty(B, w.kh, dtype=torch.int32, device="cuda")
    S = Sh = None
    if not inline:
        rng = np.random.default_rng(seed)
        S = torch.from_numpy(random_sets(rng, B, w.d_ffn, w.k)).cuda()
        Sh = torch.from_numpy(random_sets(rng, B, w.n_heads, w.kh)).cuda()
    dims = dims_of(w)
    pred = pred_weights(t) if inline else None
    if noalloc:
        dv.dv_layer_step_noalloc(dims, layer_weights(t), pred, x, x, w.k, w.kh, S, Sh, kc, vc, w.t_past, out, io, ho)
    else:
        dv.dv_layer_step(dims, layer_weights(t), pred, x, x, w.k, w.kh, S, Sh, kc, vc, w.t_past, out, io, ho,
                         ws=dv.workspace(dims, B, w.k, w.kh))
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (out, io, ho, kc, vc)]


CASES = [(W_C2, 4, True, 11), (W_RAG16, 1, False, 12)]


def test_two_calls_in_a_row_match_workspace_path(dv):
    for w, B, inline, seed in CASES:        # the second call is the smaller one
        ref = case(dv, w, B, inline, False, seed)
        got = case(dv, w, B, inline, True, seed)
        for name, a, b in zip(("x_out", "idx_out", "heads_out", "k_cache", "v_cache"), got, ref):
            assert np.array_equal(a, b), f"{w.name} B={B}: {name} differs from dv_layer_step's"


def test_oversized_request_is_refused(dv):
    w = synth.OPT175B_BATCHED.with_(batch=16)
    dims = dims_of(w)
    assert dv.dv_workspace_bytes(dims, 16, w.k, w.kh) > 32 << 20
    x = torch.zeros(16, w.d_model, device="cuda")
    with pytest.raises(dv.DejavuError) as e:
        dv.dv_layer_step_noalloc(dims, layer_weights({k: x for k in ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t",
                                                                         "b1", "w2", "b2")}),
                                 None, x, x, w.k, w.kh, torch.zeros(16, w.k, dtype=torch.int32, device="cuda"),
                                 torch.zeros(16, w.kh, dtype=torch.int32, device="cuda"), x, x, 0, x)
    assert e.value.status_name == "DV_ERR_WORKSPACE"
