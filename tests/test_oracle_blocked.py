"""Pins of the blocked-channel oracle (DejaVu Guide, "Blocked Channel Sparsity") on the CPU."""
import numpy as np
import pytest

import oracle


def test_block_one_is_identity():
    rng = np.random.default_rng(0)
    s = rng.standard_normal((3, 40)).astype(np.float32)
    assert np.array_equal(oracle.block_scores(s, 1), s)


def test_block_max_brute_force_and_bounds():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((2, 96)).astype(np.float32)
    s[0, 5] = np.nan
    s[1, 64:96] = np.nan       # a whole block of NaNs
    for bs in (2, 8, 32):
        got = oracle.block_scores(s, bs)
        for b in range(2):
            for j in range(96 // bs):
                vals = [float(v) for v in s[b, j * bs:(j + 1) * bs] if not np.isnan(v)]
                want = max(vals) if vals else -np.inf
                assert got[b, j] == np.float32(want)
                assert all(got[b, j] >= v for v in vals)


def test_blocked_selection_equals_neuron_selection_of_expanded_blocks():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((1, 64)).astype(np.float32)
    blocks = oracle.topk(oracle.block_scores(s, 8), 3)
    S = oracle.expand_blocks(blocks, 8)
    assert S.shape == (1, 24) and np.all(np.diff(S[0]) > 0)
    # every selected block holds a neuron at least as high as any unselected block's best
    bs = oracle.block_scores(s, 8)[0]
    chosen = set(blocks[0].tolist())
    assert min(bs[list(chosen)]) >= max(bs[[j for j in range(8) if j not in chosen]])
    # the argmax neuron's block is always chosen
    assert int(np.argmax(s[0])) // 8 in chosen


def test_expand_blocks_brute_force():
    blocks = np.array([[0, 3], [1, 2]], np.int32)
    assert oracle.expand_blocks(blocks, 4).tolist() == [[0, 1, 2, 3, 12, 13, 14, 15], [4, 5, 6, 7, 8, 9, 10, 11]]


def test_rejects_ragged_blocks():
    with pytest.raises(ValueError):
        oracle.block_scores(np.zeros((1, 10), np.float32), 4)
