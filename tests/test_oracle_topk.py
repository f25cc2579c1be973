"""Pins for the oracle's top-k selection (CPU only).

The selection rule (DejaVu Guide, "Mathematical Formulation of Lookahead
Predictors"; sorted indices per the predictor of "Step-by-Step
Implementation"): the k highest scores, ties to the lower index, -0.0 == +0.0,
NaN below -inf, output ascending.
"""
import itertools
import math
import random

import numpy as np
import pytest
import torch

import oracle

ALPHABET = [-math.inf, -1.0, -0.0, 0.0, 1.0, math.inf, math.nan]


def beats(vals, i, j):
    """True if element i ranks above element j, written from the rule alone."""
    a, b = vals[i], vals[j]
    na, nb = math.isnan(a), math.isnan(b)
    if na and nb:
        return i < j
    if na:
        return False
    if nb:
        return True
    if a == b:            # Python float ==: -0.0 == 0.0
        return i < j
    return a > b


def is_topk_set(vals, S):
    out = set(range(len(vals))) - set(S)
    return all(beats(vals, i, j) for i in S for j in out)


def check_exhaustive(topk_fn, n):
    for vals in itertools.product(ALPHABET, repeat=n):
        arr = np.array(vals, np.float32)
        for k in range(n + 1):
            got = list(topk_fn(arr, k)[0])
            assert got == sorted(got)
            # exactly one k-subset satisfies the characterisation, and it is the result
            valid = [S for S in itertools.combinations(range(n), k) if is_topk_set(vals, S)]
            assert len(valid) == 1, (vals, k, valid)
            assert tuple(got) == valid[0], (vals, k, got, valid)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_exhaustive_subset_characterisation(n):
    check_exhaustive(oracle.topk, n)


def test_random_length5_6_with_specials():
    rng = random.Random(7)
    for _ in range(400):
        n = rng.choice([5, 6])
        vals = [rng.choice(ALPHABET) for _ in range(n)]
        arr = np.array(vals, np.float32)
        for k in range(n + 1):
            got = tuple(oracle.topk(arr, k)[0])
            assert is_topk_set(vals, got) and len(got) == k


def py_sorted_topk(vals, k):
    def key(i):
        v = vals[i]
        if math.isnan(v):
            return (0, 0.0, i)
        return (1, -(v + 0.0), i)
    order = sorted(range(len(vals)), key=lambda i: (-key(i)[0], key(i)[1], key(i)[2]))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_sorted_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 4097))
    # few distinct values -> many ties at the k-th value
    vals = rng.integers(-4, 5, n).astype(np.float32) * 0.5
    vals[rng.random(n) < 0.05] = -0.0
    vals[rng.random(n) < 0.02] = np.nan
    for k in {0, 1, n // 3, n // 2, n - 1, n}:
        if k < 0:
            continue
        assert list(oracle.topk(vals, k)[0]) == py_sorted_topk(vals.tolist(), k)


def test_identities():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((3, 257)).astype(np.float32)
    assert np.array_equal(oracle.topk(s, 257), np.tile(np.arange(257), (3, 1)))
    assert oracle.topk(s, 0).shape == (3, 0)
    eq = np.full((2, 50), 3.25, np.float32)
    assert np.array_equal(oracle.topk(eq, 17), np.tile(np.arange(17), (2, 1)))
    # exact scaling by 2 preserves the order
    assert np.array_equal(oracle.topk(s, 40), oracle.topk(s * 2, 40))


def test_set_equality_with_torch_topk_on_distinct_values():
    rng = np.random.default_rng(3)
    s = rng.permutation(100000).astype(np.float32)[:49152].reshape(1, -1)
    k = 2458
    ref = torch.topk(torch.from_numpy(s), k, dim=-1).indices.numpy()
    assert np.array_equal(oracle.topk(s, k), np.sort(ref, axis=-1))


def test_planted_mistake_is_caught(monkeypatch):
    """A tie rule flipped to the higher index must fail the exhaustive pin."""
    def wrong(scores, k):
        s = np.atleast_2d(np.asarray(scores, np.float32))
        out = []
        for row in s:
            cls, val = oracle.topk_order_key(row)
            idx = np.arange(row.size)
            order = np.lexsort((-idx, -val, -cls))   # ties to the HIGHER index
            out.append(np.sort(order[:k]))
        return np.array(out, np.int32).reshape(s.shape[0], k)
    with pytest.raises(AssertionError):
        check_exhaustive(wrong, 3)
