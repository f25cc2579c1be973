"""Pins of the predictor-training oracle (CPU): the loss against its textbook form and limits,
the gradient against finite differences, descent, a planted low-rank problem that must be
learned, recall by hand, and the training targets against closed forms and brute force."""
import math

import numpy as np
import pytest

import oracle
import synth


def test_bce_zero_logits_is_log2():
    rng = np.random.default_rng(0)
    y = rng.integers(0, 2, (7, 5))
    assert oracle.bce_logits(np.zeros((7, 5)), y) == pytest.approx(math.log(2.0), rel=1e-15)


def test_bce_matches_textbook_form():
    rng = np.random.default_rng(1)
    s = rng.uniform(-8, 8, (6, 9))
    y = rng.integers(0, 2, (6, 9))
    ref = 0.0
    for v, t in zip(s.ravel(), y.ravel()):
        p = 1.0 / (1.0 + math.exp(-v))
        ref += -(t * math.log(p) + (1 - t) * math.log(1.0 - p))
    assert oracle.bce_logits(s, y) == pytest.approx(ref / s.size, rel=1e-12)


def test_bce_extreme_logits_are_finite_and_exact():
    s = np.array([[1000.0, -1000.0, 1000.0, -1000.0]])
    y = np.array([[1, 0, 0, 1]])
    # right with margin 1000 costs 0, wrong costs 1000
    assert oracle.bce_logits(s, y) == pytest.approx((0 + 0 + 1000 + 1000) / 4, rel=1e-15)


def test_sigmoid_values_and_symmetry():
    s = np.array([-800.0, -3.0, 0.0, 2.5, 800.0])
    g = oracle.sigmoid(s)
    assert g[2] == 0.5 and g[0] == pytest.approx(0.0, abs=1e-300) and g[4] == 1.0
    assert np.allclose(oracle.sigmoid(-s), 1.0 - g, rtol=0, atol=1e-15)
    assert g[3] == pytest.approx(1.0 / (1.0 + math.exp(-2.5)), rel=1e-15)


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(2)
    M, d, r, N = 5, 6, 3, 4
    x = rng.standard_normal((M, d))
    y = rng.integers(0, 2, (M, N))
    p1 = rng.standard_normal((r, d))
    p2 = rng.standard_normal((N, r))
    _, g1, g2 = oracle.predictor_loss_grad(x, y, p1, p2)
    h = 1e-6

    def loss(a, b):
        return oracle.bce_logits((x @ a.T) @ b.T, y)

    for P, G, which in ((p1, g1, 0), (p2, g2, 1)):
        num = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            lp = loss(Pp, p2) if which == 0 else loss(p1, Pp)
            lm = loss(Pm, p2) if which == 0 else loss(p1, Pm)
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - G)) <= 1e-8 * max(1.0, np.max(np.abs(G))), f"factor {which + 1}"


def test_small_steps_descend():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 8))
    y = rng.integers(0, 2, (40, 6))
    p1 = 0.3 * rng.standard_normal((2, 8))
    p2 = 0.3 * rng.standard_normal((6, 2))
    _, _, losses = oracle.train_predictor(x, y, p1, p2, 30, 0.05, 0.0)
    assert all(b < a for a, b in zip(losses, losses[1:]))


def test_momentum_changes_the_path_but_starts_like_plain_descent():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((30, 7))
    y = rng.integers(0, 2, (30, 5))
    p1 = 0.3 * rng.standard_normal((2, 7))
    p2 = 0.3 * rng.standard_normal((5, 2))
    a1, b1, _ = oracle.train_predictor(x, y, p1, p2, 1, 0.1, 0.9)
    a0, b0, _ = oracle.train_predictor(x, y, p1, p2, 1, 0.1, 0.0)
    assert np.array_equal(a1, a0) and np.array_equal(b1, b0)   # zero velocity at the start
    a1, _, _ = oracle.train_predictor(x, y, p1, p2, 2, 0.1, 0.9)
    a0, _, _ = oracle.train_predictor(x, y, p1, p2, 2, 0.1, 0.0)
    assert not np.allclose(a1, a0)


def test_planted_low_rank_problem_is_learned():
    """Targets made by a rank-3 linear rule are separable by the predictor's own form, so
    training from a small start must reach (almost) every target."""
    rng = np.random.default_rng(0)
    M, d, r, N = 400, 20, 3, 10
    x = rng.standard_normal((M, d))
    y = (((x @ rng.standard_normal((r, d)).T) @ rng.standard_normal((N, r)).T) > 0).astype(np.uint8)
    p1 = 0.1 * rng.standard_normal((r, d))
    p2 = 0.1 * rng.standard_normal((N, r))
    a, b, losses = oracle.train_predictor(x, y, p1, p2, 300, 3.0, 0.9)
    acc = np.mean((((x @ a.T) @ b.T) > 0) == y)
    assert losses[0] > 0.6 and losses[-1] < 0.02 and acc >= 0.99


def test_recall_by_hand():
    labels = np.array([[1, 0, 1, 0, 1], [0, 0, 0, 0, 0], [0, 1, 0, 0, 0], [1, 1, 0, 0, 0]])
    sets = np.array([[0, 2], [1, 3], [0, 2], [0, 1]])
    assert np.allclose(oracle.recall(sets, labels), [2 / 3, 1.0, 0.0, 1.0])


def _train_layer():
    w = synth.OPT125M_TRAIN.with_(batch=6)
    t = synth.layer_tensors(w)
    x = synth.lowdim_x(w, 6)
    return w, t, x


def test_labels_single_token_heads_are_value_norms():
    """With no past tokens a head's attention is over its own key alone, so o_h = v_h."""
    w, t, x = _train_layer()
    assert w.t_past == 0
    lab = oracle.layer_labels(x, t, synth.kv_cache(w, "k_cache"), synth.kv_cache(w, "v_cache"), 0, w.kh)
    xn = x.astype(np.float64)
    xn = xn / np.sqrt(np.mean(xn * xn, axis=1, keepdims=True) + 1e-5) * t["g1"].astype(np.float64)
    wv = t["wqkv"][:, 2].astype(np.float64)           # [H][dh][d]
    v = np.einsum("bd,hed->bhe", xn, wv) + t["bqkv"][:, 2].astype(np.float64)[None]
    assert np.allclose(lab["head_norm"], np.linalg.norm(v, axis=2), rtol=1e-12, atol=0)


def test_labels_fire_is_the_active_set():
    """The masked MLP on the firing set equals the dense MLP, and dropping any firing neuron
    changes it: the firing set is exactly the neurons that matter."""
    w, t, x = _train_layer()
    kc, vc = synth.kv_cache(w, "k_cache"), synth.kv_cache(w, "v_cache")
    lab = oracle.layer_labels(x, t, kc, vc, 0, w.kh)
    assert 0.03 < lab["fire"].mean() < 0.25
    F = w.d_ffn
    every = np.tile(np.arange(F), (x.shape[0], 1))
    heads = np.tile(np.arange(w.n_heads), (x.shape[0], 1))
    dense = oracle.layer(x, t, kc, vc, 0, every, heads)
    for b in range(2):
        on = np.flatnonzero(lab["fire"][b])
        r = oracle.mlp(dense["xn2"][b:b + 1], t["w1t"], t["b1"], t["w2"], t["b2"],
                       oracle.masks_from_sets(on[None], F))
        assert np.allclose(r["y_m"], dense["y_m"][b:b + 1], rtol=0, atol=1e-12)
        r2 = oracle.mlp(dense["xn2"][b:b + 1], t["w1t"], t["b1"], t["w2"], t["b2"],
                        oracle.masks_from_sets(on[1:][None], F))
        assert not np.allclose(r2["y_m"], dense["y_m"][b:b + 1], rtol=0, atol=1e-12)


def test_labels_head_targets_brute_force():
    w, t, x = _train_layer()
    lab = oracle.layer_labels(x, t, synth.kv_cache(w, "k_cache"), synth.kv_cache(w, "v_cache"), 0, w.kh)
    for b in range(x.shape[0]):
        nf = lab["head_norm"][b].astype(np.float32)
        order = sorted(range(w.n_heads), key=lambda h: (-float(nf[h]), h))
        assert list(lab["head_top"][b]) == sorted(order[: w.kh])
        assert lab["head_label"][b].sum() == w.kh and all(lab["head_label"][b][order[: w.kh]] == 1)
