"""Pins of oracle.kv_compact: hand-worked slot moves on the guide's example tree, the chain case,
an overlapping path that an in-place copy in the wrong order gets wrong, the untouched cases, and
several layers and heads moving alike."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def slot_cache(L, B, H, S, d):
    """Every element names its own (layer, sequence, head, slot): value = slot + 1000 h + 100000 b
    + 10000000 l, the same in every dimension, so a moved row is recognisable by eye."""
    l, b, h, s = np.meshgrid(np.arange(L), np.arange(B), np.arange(H), np.arange(S), indexing="ij")
    v = (s + 1000 * h + 100000 * b + 10000000 * l).astype(np.float64)
    return np.repeat(v[..., None], d, axis=-1)


def slot_of(cache, l, b, h, s):
    """The original slot held now at (l, b, h, s)."""
    return int(round(cache[l, b, h, s, 0])) % 1000


def test_guide_tree_path():
    """The guide's printed tree (root; t1a, t1b, t1c; t2a, t2b under t1a; t2d under t1b), with the
    accepted path root -> t1b -> t2d = nodes [0, 2, 6]: slot P+1 takes node 2's K/V (slot P+2),
    slot P+2 takes node 6's (slot P+6); the prefix grows by 3."""
    g = json.load(open(os.path.join(GOLDEN, "guide_tree_example.json")))
    assert g["root_to_leaf_paths"][2] == [0, 2, 6]
    P, S, d = 10, 20, 4
    k = slot_cache(1, 1, 2, S, d)
    v = -slot_cache(1, 1, 2, S, d)
    path = np.full((1, 4), -1, dtype=np.int32)
    path[0, :3] = [0, 2, 6]
    k2, v2, P2 = oracle.kv_compact(k, v, np.array([P]), path, np.array([2]))
    assert int(P2[0]) == 13
    for h in range(2):
        assert slot_of(k2, 0, 0, h, 11) == 12 and slot_of(k2, 0, 0, h, 12) == 16
        assert v2[0, 0, h, 11, 0] == -k2[0, 0, h, 11, 0]
        for s in list(range(0, 11)) + list(range(13, S)):     # every other slot as it was
            assert slot_of(k2, 0, 0, h, s) == s


def test_chain_changes_nothing_but_the_prefix():
    """On a chain the path is 0, 1, ..., a: every node already sits at its committed slot."""
    k = slot_cache(2, 3, 2, 16, 3)
    v = 2 * k
    path = np.tile(np.arange(8, dtype=np.int32), (3, 1))
    for a in range(0, 8):
        k2, v2, P2 = oracle.kv_compact(k, v, np.array([0, 3, 8]), path, np.array([a] * 3))
        assert np.array_equal(k2, k) and np.array_equal(v2, v)
        assert P2.tolist() == [a + 1, 3 + a + 1, 8 + a + 1]


def test_overlapping_path_reads_before_writing():
    """Path [0, 2, 3]: slot P+2 is both the source of node 2 (moved to P+1) and the destination
    of node 3.  Correct: P+1 <- old P+2, P+2 <- old P+3.  Copying in place in decreasing j
    order would put old P+3 into P+1."""
    k = slot_cache(1, 1, 1, 8, 2)
    path = np.array([[0, 2, 3, -1]], dtype=np.int32)
    k2, _, P2 = oracle.kv_compact(k, k.copy(), np.array([0]), path, np.array([2]))
    assert [slot_of(k2, 0, 0, 0, s) for s in range(8)] == [0, 2, 3, 3, 4, 5, 6, 7]
    assert int(P2[0]) == 3


def test_untouched_sequences():
    """accept_len 0 commits the root only; an error word, a path that does not start at the root,
    is not increasing, or reaches past the cache leave the sequence as it was."""
    S = 12
    k = slot_cache(1, 5, 1, S, 2)
    path = np.array([[0, -1, -1, -1],
                     [0, 3, 5, -1],     # error word set below
                     [1, 3, 5, -1],     # does not start at the root
                     [0, 5, 3, -1],     # not increasing
                     [0, 3, 9, -1]],    # P + 9 = 13 >= S
                    dtype=np.int32)
    P = np.array([2, 2, 2, 2, 4])
    acc = np.array([0, 2, 2, 2, 2])
    err = np.array([0, (3 << 8) | 2, 0, 0, 0])
    k2, v2, P2 = oracle.kv_compact(k, k.copy(), P, path, acc, err)
    assert np.array_equal(k2, k)
    assert P2.tolist() == [3, 2, 2, 2, 4]


def test_layers_and_heads_move_alike():
    """Three layers, four heads, two sequences with different paths and prefixes: every layer and
    head of a sequence moves the same slots; the other sequence is unaffected by it."""
    L, B, H, S, d = 3, 2, 4, 24, 5
    rng = np.random.default_rng(0)
    k = rng.standard_normal((L, B, H, S, d))
    v = rng.standard_normal((L, B, H, S, d))
    path = np.array([[0, 4, 7, 11], [0, 1, 9, -1]], dtype=np.int32)
    P = np.array([5, 9])
    acc = np.array([3, 2])
    k2, v2, P2 = oracle.kv_compact(k, v, P, path, acc)
    for (b, moves) in ((0, {6: 9, 7: 12, 8: 16}), (1, {10: 10, 11: 18})):
        for dst, src in moves.items():
            assert np.array_equal(k2[:, b, :, dst], k[:, b, :, src])
            assert np.array_equal(v2[:, b, :, dst], v[:, b, :, src])
        keep = [s for s in range(S) if s not in moves]
        assert np.array_equal(k2[:, b, :, keep], k[:, b, :, keep])
    assert P2.tolist() == [9, 12]


@pytest.mark.parametrize("a", [0, 1, 5])
def test_inputs_not_modified(a):
    k = slot_cache(1, 1, 1, 10, 2)
    kc = k.copy()
    path = np.array([[0, 2, 3, 5, 6, 8]], dtype=np.int32)
    oracle.kv_compact(k, k, np.array([1]), path, np.array([a]))
    assert np.array_equal(k, kc)
