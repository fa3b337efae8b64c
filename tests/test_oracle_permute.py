"""Pins of the oracle's grouping of (token, choice) pairs by expert."""
import numpy as np

import synth
from oracle.permute import permute


def test_hand_example():
    # flat ids [2,0 | 0,1 | 2,1]: expert 0 <- flat 1,2; expert 1 <- 3,5; expert 2 <- 0,4
    counts, offsets, perm, inv = permute(np.array([[2, 0], [0, 1], [2, 1]]), 3)
    assert counts.tolist() == [2, 2, 2]
    assert offsets.tolist() == [0, 2, 4, 6]
    assert perm.tolist() == [1, 2, 3, 5, 0, 4]
    assert inv.tolist() == [4, 0, 1, 2, 5, 3]


def test_against_bincount_and_stable_argsort():
    for T, E, k, seed in ((1, 8, 2, 0), (16, 8, 2, 1), (64, 128, 8, 2), (517, 256, 6, 3), (3000, 1024, 8, 4)):
        idx = synth.forced_topk(seed, T, E, k)
        counts, offsets, perm, inv = permute(idx, E)
        flat = idx.ravel()
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(np.sort(perm), np.arange(T * k))
        assert np.array_equal(inv[perm], np.arange(T * k))
        assert np.array_equal(flat[perm], np.repeat(np.arange(E), counts))


def test_skewed_and_degenerate():
    # all pairs on one expert; one expert per token (k = 1); k = E
    idx = np.zeros((50, 1), np.int32)
    c, o, p, i = permute(idx, 4)
    assert c.tolist() == [50, 0, 0, 0] and p.tolist() == list(range(50))
    idx = np.tile(np.arange(5, dtype=np.int32)[::-1], (7, 1))
    c, o, p, i = permute(idx, 5)
    assert c.tolist() == [7] * 5
    assert np.array_equal(p, np.argsort(idx.ravel(), kind="stable"))
