"""Shared helpers of the GPU parity tests: build seeded cases, run the oracle, compare.

Tolerances (written here, used by every GPU test):
* predictor scores: |s_gpu - s_ref| <= 1e-3 * max(|s_ref|, RMS(s_ref)) elementwise;
* top-k index sets: bit-exact on identical fp32 scores;
* layer outputs: max-abs error <= 2e-2 * RMS(ref) for fp16 weights (fp32 accumulation),
  applied separately to y_a, y_m and the layer output; and the tighter internal bars
  FP16_BAR / FP32_BAR derived from fp32 accumulation error, BATCHED_BAR where a batch of
  two or more rows runs on the matrix cores with fp16 activations.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

LAYER_TOL = 2e-2
FP16_BAR = 1e-3
FP32_BAR = 1e-4
SCORE_TOL = 1e-3
# Batched path (B >= 2, fp16 weights): activations are rounded to fp16 for the matrix cores
# (2^-11 relative per operand, through the q/k/v, attention, ReLU and both projections).
BATCHED_BAR = 4e-3

LAYER_KEYS = ("g1", "g2", "wqkv", "bqkv", "wo", "bo", "w1t", "b1", "w2", "b2")
PRED_KEYS = ("p1_mlp", "p2_mlp", "p1_head", "p2_head")

# Small parity workloads (nonzero biases, so every bias path is exercised).
W_C1 = synth.OPT125M_LAYER.with_(bias_sigma=0.02)
W_C2 = synth.OPT6P7B_LAYER.with_(bias_sigma=0.02)
# Ragged shapes: rows that do not fill a tile, odd k, short caches.
W_RAG16 = synth.Workload("ragged-f16", 6, 640, 1000, 5, 128, 72, 37, 77, 2, "f16", bias_sigma=0.02)
W_RAG32 = synth.Workload("ragged-f32", 7, 320, 999, 5, 64, 36, 19, 101, 2, "f32", bias_sigma=0.02)


def dims_of(w: synth.Workload):
    import contextual_activation_sparsity_amd as dv
    return dv.Dims(w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank, w.rank, w.t_max, w.dtype)


def to_dev(arrs):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrs.items()}


def layer_weights(t):
    import contextual_activation_sparsity_amd as dv
    return dv.LayerWeights(**{k: t[k] for k in LAYER_KEYS})


def pred_weights(t):
    import contextual_activation_sparsity_amd as dv
    return dv.PredictorWeights(**{k: t[k] for k in PRED_KEYS})


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


# Every layer-output comparison, for the end-of-run summary (conftest.py): (what, max-abs
# error / RMS(ref), internal bar it was held to).
ERRORS: list = []


def assert_close(got, ref, dtype: str, what: str, batch: int = 1, depth: int = 1):
    """Layer bar and the internal bar; `depth` layers of a chain where the oracle runs on its
    own outputs add up to `depth` single-layer errors (the residual stream carries them)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = max(rms(ref), 1e-30)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bar = FP16_BAR if dtype == "f16" else FP32_BAR
    if dtype == "f16" and batch >= 2:
        bar = BATCHED_BAR
    bar *= depth
    ERRORS.append((what, err / scale, bar))
    assert err <= LAYER_TOL * scale, f"{what}: max-abs {err:.3e} > {LAYER_TOL} * RMS {scale:.3e}"
    assert err <= bar * scale, f"{what}: max-abs {err:.3e} > internal bar {bar} * RMS {scale:.3e}"
    return err / scale


def assert_scores_close(got, ref, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rms(ref)
    bound = SCORE_TOL * np.maximum(np.abs(ref), r)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} scores off, worst {np.max(np.abs(got - ref) / bound):.3f}x bound"


def random_sets(rng, B: int, n: int, k: int) -> np.ndarray:
    return np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32) \
        if k > 0 else np.zeros((B, 0), np.int32)


def kv_host(w: synth.Workload, which: str, layer: int = 0) -> np.ndarray:
    return synth.kv_cache(w, which, layer)


def compact_layer(w: synth.Workload, layer: int, S: np.ndarray, Sh: np.ndarray, b: int):
    """Selected rows of one layer's weights and row b's caches, regenerated on the host.

    The oracle on these compacted arrays with all-ones masks equals the masked dense
    oracle (pinned on the CPU); it avoids drawing the unselected rows of large layers.
    """
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
    kvs = []
    for which in ("k_cache", "v_cache"):
        shp = (w.batch * w.n_heads, w.t_max, w.head_dim)
        r = synth.rows(w.key(which, layer), shp, w.kv_sigma, w.dtype, b * w.n_heads + np.asarray(Sh))
        r[:, w.t_past:, :] = 0
        kvs.append(r[None])
    return t, kvs[0], kvs[1]


def oracle_layer_compact(w, layer, x_b, S, Sh, b):
    t, kc, vc = compact_layer(w, layer, S, Sh, b)
    return oracle.layer(x_b[None], t, kc, vc, w.t_past, [np.arange(len(S))], [np.arange(len(Sh))])


def predictor_host(w, layer):
    shapes = synth.layer_shapes(w)
    return {n: synth.tensor(w.key(n, layer), *shapes[n]) for n in PRED_KEYS}


# Every chained comparison of selected sets, for the end-of-run summary (conftest.py):
# (what, row, k, indices in one set but not the other, oracle scores inside the tie band).
SET_DRIFT: list = []


def max_swaps(k: int) -> int:
    """Near-tie swaps a row may show: one, or one per 200 selected indices for long lists.
    The GPU's fp32 scores sit about 1e-6 relative from the oracle's, so a swap needs two
    scores that close around the k-th; more swaps than this mean the score error grew."""
    return max(1, k // 200)


def sets_match(got, scores_ref, k: int, what: str) -> bool:
    """The GPU's selected sets [B][k] against the oracle's own selection on its own scores.

    The selection is an integer decision taken in fp32 on both sides. Where the GPU's set
    differs from the oracle's, every index in one set but not the other must sit at a near
    tie: its oracle score within twice the score bar of the k-th largest, so that either
    choice is a correct top-k within the precision of the scores; and the row may differ by
    at most max_swaps(k) swaps. Every row's difference count is recorded in SET_DRIFT.
    Returns True when every row's set equals the oracle's.
    """
    got = np.atleast_2d(np.asarray(got))
    scores_ref = np.atleast_2d(np.asarray(scores_ref, np.float64))
    ref = oracle.topk(scores_ref.astype(np.float32), k)
    same = True
    for b in range(got.shape[0]):
        assert len(set(got[b].tolist())) == k, f"{what} row {b}: repeated indices"
        s = scores_ref[b]
        kth = np.sort(s)[::-1][k - 1] if k > 0 else 0.0
        band = 2 * SCORE_TOL * max(abs(kth), rms(s))
        in_band = int(np.count_nonzero(np.abs(s - kth) <= band)) if k > 0 else 0
        if np.array_equal(got[b], ref[b]):
            SET_DRIFT.append((what, b, k, 0, in_band))
            continue
        same = False
        diff = set(got[b].tolist()) ^ set(ref[b].tolist())
        SET_DRIFT.append((what, b, k, len(diff), in_band))
        assert all(abs(s[j] - kth) <= band for j in diff), \
            f"{what} row {b}: sets differ away from the k-th score ({sorted(diff)[:8]})"
        assert len(diff) <= 2 * max_swaps(k), \
            f"{what} row {b}: {len(diff) // 2} near-tie swaps, more than {max_swaps(k)} (score error grew?)"
    return same


def chosen_sets(got, scores_ref, k: int, what: str):
    """The sets a chained oracle continues with: its own top-k, or, where the GPU took the
    other side of a near tie (validated by sets_match), the GPU's equally correct choice."""
    return oracle.topk(np.asarray(scores_ref, np.float64).astype(np.float32), k) \
        if sets_match(got, scores_ref, k, what) else np.atleast_2d(np.asarray(got))
