"""fp64 definitions of predictor training: labels from the dense layer, the loss and its
gradient for the rank-r score map, gradient descent, and recall of the selected sets.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "DejaVu Guide: Contextual Sparsity for LLM Inference", "Mathematical Formulation of
  Lookahead Predictors": the head predictor's target marks the heads that carry the
  top-k attention norms; the neuron predictor's target marks the MLP neurons that fire;
  both predictors read the layer input.
* "Deja Vu: How Contextual Sparsity Accelerates LLM Inference by 6x", "What Is
  Contextual Sparsity?" (offline phase): run the dense model, record which heads and
  neurons each input activates, and train a small classifier per layer on the layer's
  input to predict them.

The pages name neither the loss nor the optimiser. The reading taken here: each score is
the logit of an independent binary classifier, trained on the mean binary cross-entropy
over all (sample, neuron) pairs by full-batch gradient descent with heavy-ball momentum.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

from .dejavu import layer, mlp, topk


def _f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64)


def layer_labels(x, t: Dict[str, np.ndarray], k_cache, v_cache, t_past: int, kh: int) -> Dict[str, np.ndarray]:
    """Training targets of one layer for a batch of inputs, from the dense layer.

    The dense layer is the sparse layer with every head and every neuron selected.
    * neuron j fires for a row when its up-projection pre-activation a_j (on the
      normalised MLP input, bias included) is positive, i.e. when ReLU passes it;
    * the norm of head h is ||o_h||_2, the Euclidean norm of the head's attention output
      (before the output projection);
    * the head targets are the kh heads of largest norm (the selection's tie rule: the
      lower index wins), with the norms rounded to fp32 first, the precision the kernels
      decide in.

    Returns fire [B][F] uint8, a [B][F], head_norm [B][H], head_top [B][kh] (ascending)
    and head_label [B][H] uint8.
    Pins: with no past tokens o_h is the head's value vector; the masked MLP on the
    firing set equals the dense MLP and dropping any firing neuron changes it; head
    targets by brute force over sorted().
    """
    x = _f64(x)
    B = x.shape[0]
    H = np.shape(t["wqkv"])[0]
    F = np.shape(t["w1t"])[0]
    every_head = np.tile(np.arange(H), (B, 1))
    every_neuron = np.tile(np.arange(F), (B, 1))
    out = layer(x, t, k_cache, v_cache, t_past, every_neuron, every_head)
    a = mlp(out["xn2"], t["w1t"], t["b1"], t["w2"], t["b2"], np.ones((B, F)))["a"]
    fire = (a > 0.0).astype(np.uint8)
    head_norm = np.sqrt(np.sum(out["o"] ** 2, axis=-1))
    head_top = topk(head_norm.astype(np.float32), kh)
    head_label = np.zeros((B, H), np.uint8)
    for b in range(B):
        head_label[b, head_top[b]] = 1
    return {"fire": fire, "a": a, "head_norm": head_norm, "head_top": head_top, "head_label": head_label}


def sigmoid(s) -> np.ndarray:
    """Logistic function, evaluated without overflow for either sign."""
    s = _f64(s)
    e = np.exp(-np.abs(s))
    return np.where(s >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def bce_logits(s, y) -> float:
    """Mean binary cross-entropy of logits s against 0/1 targets y.

    Per element -y log sigmoid(s) - (1 - y) log(1 - sigmoid(s)), evaluated as
    softplus(s) - y s with softplus(s) = max(s, 0) + log(1 + e^-|s|).
    Pins: zero logits give log 2; the textbook form on moderate logits; the limits at
    very large |s|.
    """
    s = _f64(s)
    y = _f64(y)
    softplus = np.maximum(s, 0.0) + np.log1p(np.exp(-np.abs(s)))
    return float(np.mean(softplus - y * s))


def predictor_loss_grad(x, y, p1, p2) -> Tuple[float, np.ndarray, np.ndarray]:
    """Loss and gradients of the rank-r score map under the mean cross-entropy.

    Scores s = (x . P1^T) . P2^T for x [M][d], P1 [r][d], P2 [N][r]; targets y [M][N].
    With z = x . P1^T and G = dL/ds = (sigmoid(s) - y) / (M N):
    dL/dP2 = G^T . z,  dL/dz = G . P2,  dL/dP1 = (dL/dz)^T . x.
    Returns (loss, dL/dP1 [r][d], dL/dP2 [N][r]).
    Pins: central finite differences on every parameter of a small problem.
    """
    x, y, p1, p2 = _f64(x), _f64(y), _f64(p1), _f64(p2)
    M, N = y.shape
    z = x @ p1.T
    s = z @ p2.T
    loss = bce_logits(s, y)
    g = (sigmoid(s) - y) / (M * N)
    g2 = g.T @ z
    gz = g @ p2
    g1 = gz.T @ x
    return loss, g1, g2


def train_predictor(x, y, p1, p2, steps: int, lr: float, momentum: float
                    ) -> Tuple[np.ndarray, np.ndarray, List[float]]:
    """Full-batch gradient descent with heavy-ball momentum.

    Velocities start at zero; each step computes the gradient at the current parameters,
    then v <- momentum * v + grad and P <- P - lr * v, for both factors.
    Returns the final (P1, P2) and the loss before each step's update.
    Pins: the loss descends for a small step size; a planted rank-r problem is learned.
    """
    p1, p2 = _f64(p1).copy(), _f64(p2).copy()
    v1, v2 = np.zeros_like(p1), np.zeros_like(p2)
    losses = []
    for _ in range(steps):
        loss, g1, g2 = predictor_loss_grad(x, y, p1, p2)
        losses.append(loss)
        v1 = momentum * v1 + g1
        v2 = momentum * v2 + g2
        p1 = p1 - lr * v1
        p2 = p2 - lr * v2
    return p1, p2, losses


def recall(pred_sets, labels) -> np.ndarray:
    """Share of each row's positive targets that its selected set contains.

    pred_sets [B][k] index lists, labels [B][n] 0/1; a row with no positive target has
    recall 1. Pins: by hand on small cases (exact, disjoint, partial, empty).
    """
    pred_sets = np.atleast_2d(np.asarray(pred_sets, np.int64))
    labels = np.atleast_2d(np.asarray(labels))
    out = np.empty(labels.shape[0])
    for b in range(labels.shape[0]):
        pos = set(np.flatnonzero(labels[b]).tolist())
        out[b] = 1.0 if not pos else len(pos & set(pred_sets[b].tolist())) / len(pos)
    return out
