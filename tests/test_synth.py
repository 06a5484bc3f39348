"""Checks of the seeded input generator (shapes, distributions, routing)."""
import numpy as np

import synth


def test_dense_recipe_and_determinism():
    a = synth.dense_workload(**synth.DENSE_SMALL, seed=0)
    b = synth.dense_workload(**synth.DENSE_SMALL, seed=0)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    x = synth.bf16_bits_to_f32(a["x"])
    w = synth.bf16_bits_to_f32(a["w"])
    assert x.shape == (64, 1024) and w.shape == (1024, 1024)
    col_rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=0))
    assert (col_rms > 8).sum() == 8                      # eight outlier channels at x20
    assert abs(w.std() - 0.02) < 5e-4


def test_routing_recipe():
    ids, w = synth.routing(np.random.default_rng(0), 4096, 64, 8)
    assert ids.shape == (4096, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids[:200])
    assert np.allclose(w.sum(axis=1), 1, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    counts = np.bincount(ids.ravel(), minlength=64)
    assert counts.sum() == 4096 * 8 and counts.max() > 3000   # Zipf-skewed load
