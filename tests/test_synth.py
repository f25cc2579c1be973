"""Checks of the seeded input generator (CPU only)."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # The first outputs of a SplitMix64 stream seeded with 0.
    got = [int(v) for v in synth.raw_bits(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_row_random_access_equals_full_tensor():
    key = synth.stream_key(0, 9, 3, 11)
    full = synth.tensor(key, (40, 24), 0.02, "f16")
    part = synth.tensor(key, (40, 24), 0.02, "f16", row_start=17, n_rows=5)
    np.testing.assert_array_equal(full[17:22], part)
    np.testing.assert_array_equal(synth.rows(key, (40, 24), 0.02, "f16", [3, 39, 0]), full[[3, 39, 0]])


def test_moments_and_bounds():
    v = synth.normal_f32(synth.stream_key(1, 2, 3, 4), 0, 1 << 20, 0.02).astype(np.float64)
    assert abs(v.mean()) < 1e-4
    assert abs(v.std() - 0.02) < 2e-4
    assert np.max(np.abs(v)) <= 0.02 * np.sqrt(12.0) + 1e-6   # Irwin-Hall(4) support


def test_distinct_streams():
    a = synth.raw_bits(synth.stream_key(0, 4, 0, 11), 0, 64)
    b = synth.raw_bits(synth.stream_key(0, 4, 1, 11), 0, 64)
    c = synth.raw_bits(synth.stream_key(0, 4, 0, 13), 0, 64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_kv_cache_future_slots_zero():
    w = synth.OPT125M_LAYER.with_(t_past=5, n_heads=2, head_dim=8)
    kc = synth.kv_cache(w, "k_cache")
    assert kc.shape == (1, 2, 6, 8)
    assert np.all(kc[:, :, 5:] == 0) and np.any(kc[:, :, :5] != 0)


def test_zipf_scores_shape_and_skew():
    w = synth.OPT175B_BATCHED.with_(batch=4)
    s = synth.zipf_scores(w, 4096, "sel_mlp")
    assert s.shape == (4, 4096) and np.all(np.isfinite(s))
    top = np.argsort(-s, axis=1)[:, :205]
    u, cnt = np.unique(top, return_counts=True)
    assert len(u) < 4 * 205          # popular items repeat across rows
