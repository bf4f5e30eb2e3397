"""Pins for the oracle's permute (expert histogram, exclusive scan, stable
scatter): invariants, and numpy's stable argsort as an independent library
brute force."""
import numpy as np
import pytest

from oracle import moe


def _check(ids, E):
    counts, offsets, src, dest = moe.permute(ids, E)
    flat = ids.reshape(-1)
    R = flat.size
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert sorted(src.tolist()) == list(range(R))                 # bijection
    np.testing.assert_array_equal(dest[src], np.arange(R))        # dest o src = id
    np.testing.assert_array_equal(src, np.argsort(flat, kind="stable"))
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


@pytest.mark.parametrize("T,k,E", [(32, 8, 256), (64, 2, 8), (100, 1, 3), (1, 8, 8)])
def test_permute_random(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _check(ids, E)


def test_permute_worked_example_size():
    # 32 sequences x top-8 of 256 experts: 256 token-expert assignments
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(256, 8, replace=False) for _ in range(32)]).astype(np.int32)
    counts, offsets, src, dest = moe.permute(ids, 256)
    assert counts.sum() == 256 == offsets[-1] == src.size


def test_permute_skew_and_empty():
    ids = np.zeros((50, 1), dtype=np.int32)      # every token to expert 0
    _check(ids, 16)
    ids = np.tile(np.array([[5, 3]], dtype=np.int32), (40, 1))
    _check(ids, 8)
    counts, offsets, src, dest = moe.permute(np.zeros((0, 4), dtype=np.int32), 8)
    assert counts.sum() == 0 and src.size == 0 and (offsets == 0).all()
