"""Blocked-channel sparsity (DejaVu Guide, "Blocked Channel Sparsity") against the oracle (GPU):
block scores bit-exact, the blocked MLP against the dense-with-mask MLP on the expanded
neuron sets, and the whole chain scores -> block scores -> top-k -> blocked MLP."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import W_C2, W_RAG16, assert_close, dims_of, layer_weights, rms, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,bs", [(64, 1), (1024, 4), (1000, 8), (16384, 32), (49152, 64), (96, 96)])
@pytest.mark.parametrize("kind", ["normal", "ties", "specials"])
def test_block_scores_bitexact(dv, n, bs, kind):
    rng = np.random.default_rng(n + bs)
    B = 3
    s = rng.standard_normal((B, n)).astype(np.float32)
    if kind == "ties":
        s = (rng.integers(-2, 3, (B, n)) * 0.5).astype(np.float32)
    elif kind == "specials":
        m = rng.random((B, n))
        s[m < 0.1] = np.nan
        s[(m >= 0.1) & (m < 0.15)] = -np.inf
        s[(m >= 0.15) & (m < 0.2)] = np.inf
        s[(m >= 0.2) & (m < 0.3)] = -0.0
        s[1, :bs] = np.nan   # a block of NaNs
    sd = torch.from_numpy(s).cuda()
    out = torch.empty(B, n // bs, device="cuda")
    dv.dv_block_scores(sd, bs, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.block_scores(s, bs)
    # max of floats is exact; -0.0 and +0.0 compare equal
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("w,bs", [(W_C2, 32), (W_C2, 64), (W_RAG16, 8)], ids=["c2-32", "c2-64", "ragged-8"])
def test_blocked_mlp_matches_expanded_oracle(dv, w, bs):
    t = synth.layer_tensors(w)
    rng = np.random.default_rng(bs)
    B = 2
    F = w.d_ffn
    kb = max(1, w.k // bs)
    blocks = np.stack([np.sort(rng.choice(F // bs, kb, replace=False)) for _ in range(B)]).astype(np.int32)
    xn = rng.standard_normal((B, w.d_model)).astype(np.float32)
    d = to_dev({k: t[k] for k in ("w1t", "b1", "w2", "b2", "wqkv", "bqkv", "wo", "bo", "g1", "g2")})
    dims = dims_of(w)
    y = torch.empty(B, w.d_model, device="cuda")
    ws = dv.workspace(dims, B, kb * bs, 0)
    dv.dv_sparse_mlp_blocked(dims, layer_weights(d), torch.from_numpy(xn).cuda(), torch.from_numpy(blocks).cuda(), kb,
                             bs, y, ws)
    torch.cuda.synchronize()
    S = oracle.expand_blocks(blocks, bs)
    ref = oracle.mlp(xn, t["w1t"], t["b1"], t["w2"], t["b2"], oracle.masks_from_sets(S, F))["y_m"]
    assert_close(y.cpu().numpy(), ref, w.dtype, f"blocked y_m bs={bs}")


def test_blocked_chain_scores_to_mlp(dv):
    """GPU predictor scores -> block scores -> top-k of blocks -> blocked MLP, each step
    against the oracle on the same inputs (bit-exact selection on identical scores)."""
    w = W_C2
    t = synth.layer_tensors(w)
    bs = 64
    kb = w.k // bs
    rng = np.random.default_rng(3)
    s = (rng.standard_normal((1, w.d_ffn)) * 4).astype(np.float32)
    sd = torch.from_numpy(s).cuda()
    bsc = torch.empty(1, w.d_ffn // bs, device="cuda")
    dv.dv_block_scores(sd, bs, bsc)
    blocks = torch.empty(1, kb, dtype=torch.int32, device="cuda")
    dv.dv_topk(bsc, kb, blocks)
    torch.cuda.synchronize()
    ref_blocks = oracle.topk(oracle.block_scores(s, bs), kb)
    assert np.array_equal(blocks.cpu().numpy(), ref_blocks)
    xn = rng.standard_normal((1, w.d_model)).astype(np.float32)
    d = to_dev({k: t[k] for k in ("w1t", "b1", "w2", "b2", "wqkv", "bqkv", "wo", "bo", "g1", "g2")})
    dims = dims_of(w)
    y = torch.empty(1, w.d_model, device="cuda")
    dv.dv_sparse_mlp_blocked(dims, layer_weights(d), torch.from_numpy(xn).cuda(), blocks, kb, bs, y,
                             dv.workspace(dims, 1, kb * bs, 0))
    torch.cuda.synchronize()
    S = oracle.expand_blocks(ref_blocks, bs)
    ref = oracle.mlp(xn, t["w1t"], t["b1"], t["w2"], t["b2"], oracle.masks_from_sets(S, w.d_ffn))["y_m"]
    assert_close(y.cpu().numpy(), ref, w.dtype, "blocked chain y_m")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bs", [32, 64])
def test_blocked_mlp_opt175b_shape(dv, bs):
    """The blocked MLP at the OPT-175B shape the blocked bench times (d 12288, F 49152, 5 % of
    the neurons as 77 blocks of 32 or 38 blocks of 64), batch 1: y_m against the oracle on the
    regenerated rows of the selected blocks."""
    import synth.device as sdev
    w = synth.OPT175B_STACK
    F = w.d_ffn
    kb = (w.k + bs // 2) // bs
    rng = np.random.default_rng(100 + bs)
    blocks = np.sort(rng.choice(F // bs, kb, replace=False)).astype(np.int32)[None]
    xn = rng.standard_normal((1, w.d_model)).astype(np.float32)
    t = sdev.layer_on_device(w, 0)
    dims = dims_of(w)
    y = torch.empty(1, w.d_model, device="cuda")
    dv.dv_sparse_mlp_blocked(dims, layer_weights(t), torch.from_numpy(xn).cuda(), torch.from_numpy(blocks).cuda(), kb,
                             bs, y, dv.workspace(dims, 1, kb * bs, 0))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    del t
    torch.cuda.empty_cache()
    S = oracle.expand_blocks(blocks, bs)[0]
    shapes = synth.layer_shapes(w)
    rows = {n: synth.rows(w.key(n, 0), *shapes[n], S) for n in ("w1t", "b1", "w2")}
    b2 = synth.tensor(w.key("b2", 0), *shapes["b2"])
    ref = oracle.mlp(xn, rows["w1t"], rows["b1"], rows["w2"], b2, np.ones((1, len(S))))["y_m"]
    assert_close(got, ref, w.dtype, f"OPT-175B-shaped blocked y_m bs={bs}")

