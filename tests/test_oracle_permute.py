"""Pins of the oracle's token -> expert permutation: brute-force stable sort and
the permutation invariants."""

import numpy as np
import pytest


def brute(ids, E):
    T, k = ids.shape
    pairs = sorted(range(T * k), key=lambda q: (ids.flat[q], q))
    counts = np.bincount(ids.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return offsets, np.array(pairs)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (4, 8, 2), (16, 128, 8), (33, 5, 5),
                                   (300, 64, 4), (0, 8, 2)])
def test_permute_matches_brute_force(ref, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    ids = ids.astype(np.int32)
    off, sp, inv = ref.permute(ids, E)
    boff, bsp = brute(ids, E)
    assert np.array_equal(off, boff)
    assert np.array_equal(sp, bsp)
    P = T * k
    assert off[0] == 0 and off[-1] == P and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(sp), np.arange(P))
    assert np.array_equal(sp[inv], np.arange(P))            # inv o sorted = identity
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(ids.ravel()[seg] == e)
        assert np.all(np.diff(seg // k) > 0)                 # tokens strictly ascending


def test_permute_skewed_duplicates_allowed(ref):
    """Ids need not be distinct within a token: the permutation is a pure
    counting sort of pairs."""
    ids = np.array([[2, 2], [0, 2], [2, 1]], np.int32)
    off, sp, inv = ref.permute(ids, 3)
    assert list(off) == [0, 1, 2, 6]
    assert list(sp) == [2, 5, 0, 1, 3, 4]
    assert list(inv) == [2, 3, 0, 4, 5, 1]


def test_permute_rejects_bad_ids(ref):
    with pytest.raises(ValueError):
        ref.permute(np.array([[0, 3]], np.int32), 3)
    with pytest.raises(ValueError):
        ref.permute(np.array([[-1, 0]], np.int32), 3)
