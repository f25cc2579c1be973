"""fp64 dense-with-mask definitions of the sparse decoder-layer step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Storage conventions (the same arrays the HIP library receives; the oracle only
reads them):

* ``x``            [B][d]            layer input (residual stream)
* ``p1_mlp``       [r][d]            predictor stage-1 factor, MLP
* ``p2_mlp``       [F][r]            predictor stage-2 factor, MLP (row j scores neuron j)
* ``p1_head``      [r][d], ``p2_head`` [H][r]   the same for heads
* ``wqkv``         [H][3][dh][d]     row (h, m, e) maps x to element e of q/k/v (m=0/1/2) of head h
* ``bqkv``         [H][3][dh]
* ``wo``           [H][dh][d]        row (h, e) is the output-projection row of o_h[e]
* ``w1t``          [F][d]            row j is column j of W1 (x . W1[:, j])
* ``w2``           [F][d]            row j is row j of W2
* ``k_cache``, ``v_cache``  [B][H][t_max][dh], slots 0..t_past-1 hold the past

In the pages' row-vector notation: a = x . W1 is ``w1t @ x``, and u . W2 is
``u @ w2``.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence, Tuple

import numpy as np

RMS_EPS = 1e-5


def _f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64)


# ---------------------------------------------------------------------------
# Predictor and selection
# ---------------------------------------------------------------------------

def predict(p1_mlp, p2_mlp, p1_head, p2_head, x_pred) -> Tuple[np.ndarray, np.ndarray]:
    """Low-rank lookahead predictor scores.

    DejaVu Guide, "Mathematical Formulation of Lookahead Predictors": one
    linear map from the predictor input to a score per MLP neuron and per
    head, then top-k. The map is stored as two bias-free factors with no
    nonlinearity between them (rank r), so the score of neuron j is
    sum_i p2_mlp[j, i] * (p1_mlp[i, :] . x_pred). No sigmoid is applied: it is
    monotone and would not change the top-k.

    Returns (s_mlp [B][F], s_head [B][H]).
    Pins: brute-force loops on tiny shapes; associativity against the
    collapsed single projection; identity first factor; linearity.
    """
    x = _f64(x_pred)
    z_m = x @ _f64(p1_mlp).T            # [B][r]
    z_h = x @ _f64(p1_head).T
    return z_m @ _f64(p2_mlp).T, z_h @ _f64(p2_head).T


def topk_order_key(scores) -> Tuple[np.ndarray, np.ndarray]:
    """The total order used for selection: (class, value) per element.

    class 1 for numbers, 0 for NaN (NaN ranks below -inf); value has -0.0
    and +0.0 equal. Among equal keys the lower index ranks higher.
    """
    s = np.asarray(scores, dtype=np.float64)
    cls = np.where(np.isnan(s), 0, 1)
    val = np.where(np.isnan(s), 0.0, s) + 0.0   # -0.0 + 0.0 == +0.0
    return cls, val


def topk(scores, k: int) -> np.ndarray:
    """Indices of the k highest scores of each row, returned ascending.

    DejaVu Guide, "Mathematical Formulation of Lookahead Predictors" and the
    predictor of "Step-by-Step Implementation": the active set is the top-k of
    the predictor scores; the sketch's docstring asks for the indices sorted.
    Ties go to the lower index, -0.0 equals +0.0, NaN ranks below -inf, and
    exactly k indices are returned for every k in [0, n].

    Pins: exhaustive subset characterisation on tiny alphabets with ties and
    special values; brute force by Python's sorted(); closed-form identities
    (k = n, k = 0, all-equal rows).
    """
    s = np.atleast_2d(np.asarray(scores, dtype=np.float32))
    B, n = s.shape
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    out = np.empty((B, k), np.int32)
    for b in range(B):
        cls, val = topk_order_key(s[b])
        idx = np.arange(n)
        # lexsort: last key is primary -> class desc, value desc, index asc
        order = np.lexsort((idx, -val, -cls))
        out[b] = np.sort(order[:k])
    return out


def block_scores(scores, block: int) -> np.ndarray:
    """Score of every block of `block` consecutive neurons: the largest member score.

    DejaVu Guide, "Blocked Channel Sparsity": neurons are grouped into
    contiguous blocks and a block is loaded whole when it holds a highly
    active neuron, so a block ranks by its best member. NaN members count as
    lowest (a block of NaNs scores -inf). n must be a multiple of block.
    Pins: block = 1 is the identity; brute force by Python's max(); a block's
    score bounds every member's.
    """
    s = np.atleast_2d(np.asarray(scores, dtype=np.float32))
    B, n = s.shape
    if block < 1 or n % block:
        raise ValueError("n must be a positive multiple of block")
    s = np.where(np.isnan(s), -np.inf, s)
    return s.reshape(B, n // block, block).max(axis=2).astype(np.float32)


def expand_blocks(blocks, block: int) -> np.ndarray:
    """Neuron indices of the selected blocks [B][kb] -> [B][kb * block], ascending."""
    b = np.atleast_2d(np.asarray(blocks, dtype=np.int64))
    out = (b[:, :, None] * block + np.arange(block)[None, None, :]).reshape(b.shape[0], -1)
    return np.sort(out, axis=1).astype(np.int32)


def masks_from_sets(sets, n: int) -> np.ndarray:
    """0/1 masks [B][n] from index lists [B][k]."""
    sets = np.atleast_2d(np.asarray(sets, dtype=np.int64))
    m = np.zeros((sets.shape[0], n), np.float64)
    for b in range(sets.shape[0]):
        m[b, sets[b]] = 1.0
    return m


# ---------------------------------------------------------------------------
# Layer pieces
# ---------------------------------------------------------------------------

def rmsnorm(x, g, eps: float = RMS_EPS) -> np.ndarray:
    """RMSNorm of each row: g * x / sqrt(mean(x^2) + eps).

    DejaVu Guide, "Step-by-Step Implementation": the layer sketch normalises
    the input with an RMSNorm before the sparse MLP. eps = 1e-5 and gain g.
    Pins: constant rows, scaling invariance, brute-force loop.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(g) * x / np.sqrt(ms + eps)


def qkv_all_heads(xn, wqkv, bqkv) -> np.ndarray:
    """q, k, v of every head: [B][H][3][dh] = xn . W_{q,k,v}^h + b.

    Computed for every head; the head mask is applied afterwards
    (dense with mask).
    """
    xn = _f64(xn)
    W = _f64(wqkv)
    return np.einsum("hmed,bd->bhme", W, xn) + _f64(bqkv)[None]


def attention(xn, wqkv, bqkv, wo, bo, k_cache, v_cache, t_past: int, head_mask
              ) -> Dict[str, np.ndarray]:
    """Head-masked decode attention and output projection.

    DejaVu Guide, "Head-Pruned Attention Dispatch": a head predicted inactive
    contributes nothing: its q/k/v and output-projection weights and its past
    KV entries are not used. For an active head h, the query attends over the
    t_past cached keys plus the current token's key:
    p = softmax(K q / sqrt(dh)), o_h = p^T V; inactive heads have o_h = 0.
    y_a = sum_h o_h . Wo_h + bo (no residual here).

    head_mask: [B][H] 0/1. Returns dict with y_a [B][d], o [B][H][dh],
    qkv [B][H][3][dh] (every head) and p (per active head, for inspection).
    Pins: T = 0 gives o = v; equal keys give the mean of V; empty set gives bo;
    per-head additivity; brute-force loops.
    """
    xn = _f64(xn)
    B = xn.shape[0]
    H, _, dh, d = np.shape(wqkv)
    qkv = qkv_all_heads(xn, wqkv, bqkv)
    Kc = _f64(k_cache)
    Vc = _f64(v_cache)
    m = np.asarray(head_mask, np.float64)
    o = np.zeros((B, H, dh))
    for b in range(B):
        for h in range(H):
            if m[b, h] == 0.0:
                continue
            q, kk, vv = qkv[b, h, 0], qkv[b, h, 1], qkv[b, h, 2]
            K = np.vstack([Kc[b, h, :t_past], kk[None]])
            V = np.vstack([Vc[b, h, :t_past], vv[None]])
            s = K @ q / math.sqrt(dh)
            e = np.exp(s - s.max())
            p = e / e.sum()
            o[b, h] = p @ V
    o = o * m[:, :, None]
    y_a = np.einsum("bhe,hed->bd", o, _f64(wo)) + _f64(bo)[None]
    return {"y_a": y_a, "o": o, "qkv": qkv}


def mlp(xn, w1t, b1, w2, b2, neuron_mask) -> Dict[str, np.ndarray]:
    """Neuron-masked ReLU MLP: y = (m * relu(x . W1 + b1)) . W2 + b2.

    DejaVu Guide, "The Synchronous Prediction Dilemma" (FFN = act(x W1) W2)
    and the sparse MLP of "Step-by-Step Implementation" (only the active
    columns of W1 and rows of W2 take part). Pre-activations are computed for
    every neuron and the mask zeroes the inactive ones (dense with mask).

    neuron_mask: [B][F] 0/1. Returns y_m [B][d] (no residual), a (pre-act)
    and u (masked activations).
    Pins: all-ones mask is the textbook dense MLP; the ReLU-positive set (or any
    superset) reproduces it; empty set gives b2; homogeneity with b1 = 0;
    brute force over all subsets for tiny F.
    """
    xn = _f64(xn)
    a = xn @ _f64(w1t).T + _f64(b1)[None]            # [B][F]
    u = np.asarray(neuron_mask, np.float64) * np.maximum(a, 0.0)
    y = u @ _f64(w2) + _f64(b2)[None]
    return {"y_m": y, "a": a, "u": u}


def layer(x, t: Dict[str, np.ndarray], k_cache, v_cache, t_past: int,
          neuron_sets, head_sets, eps: float = RMS_EPS) -> Dict[str, np.ndarray]:
    """One sparse decoder layer for given active sets.

    DejaVu Guide, "Step-by-Step Implementation" (the layer: pre-norm, sparse
    block, residual) with the attention block also restricted to the active
    heads, which the sketch states production does: h1 = x + Attn_Sh(norm1(x)),
    out = h1 + MLP_S(norm2(h1)).

    Returns out, h1, y_a, y_m, xn1, xn2 and the per-head k/v of the current
    token (qkv).
    """
    x = _f64(x)
    H = np.shape(t["wqkv"])[0]
    F = np.shape(t["w1t"])[0]
    xn1 = rmsnorm(x, t["g1"], eps)
    att = attention(xn1, t["wqkv"], t["bqkv"], t["wo"], t["bo"], k_cache, v_cache, t_past,
                    masks_from_sets(head_sets, H))
    h1 = x + att["y_a"]
    xn2 = rmsnorm(h1, t["g2"], eps)
    ff = mlp(xn2, t["w1t"], t["b1"], t["w2"], t["b2"], masks_from_sets(neuron_sets, F))
    return {"out": h1 + ff["y_m"], "h1": h1, "y_a": att["y_a"], "y_m": ff["y_m"],
            "xn1": xn1, "xn2": xn2, "qkv": att["qkv"], "o": att["o"], "u": ff["u"]}
