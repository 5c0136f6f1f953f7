"""Pins of oracle.tree_select: a hand-worked selection on the guide's example tree (with ties), the
objective by brute force (the kept tree has the largest sum of cumulative probabilities among all
subsets of its size, and is ancestor-closed), exact path products against rational arithmetic, the
identity, chain and nesting cases, carried tokens and rows, and the error rules."""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_pool(rng, C, max_children=None, denom=8):
    """A random candidate tree (node i attaches to a uniform earlier node) with dyadic
    probabilities k / denom, so that every path product and every sum is exact in float64."""
    parents = np.full(C, -1, dtype=np.int32)
    for i in range(1, C):
        parents[i] = rng.integers(0, i)
    prob = rng.integers(0, denom + 1, size=C).astype(np.float32) / np.float32(denom)
    return parents, prob


def exact_value(parents, prob, i):
    v = Fraction(1)
    while i > 0:
        v *= Fraction(float(prob[i]))
        i = int(parents[i])
    return v


def test_guide_tree_by_hand():
    g = json.load(open(os.path.join(GOLDEN, "select_example.json")))
    par = np.array([g["parents"]], dtype=np.int32)
    prob = np.array([g["prob"]], dtype=np.float32)
    tokens = np.array([[100 + i for i in range(7)]], dtype=np.int32)
    rows = np.array([[-1, 0, 0, 0, 1, 1, 2]], dtype=np.int32)
    for i, v in enumerate(g["values"]):
        assert oracle.path_value(par[0], prob[0], i) == v
    for N_str, want in g["kept"].items():
        N = int(N_str)
        r = oracle.tree_select(par, prob, N, cand_tokens=tokens, cand_row=rows)
        n = len(want["sel"])
        assert int(r["n_nodes"][0]) == n and int(r["err"][0]) == 0
        assert r["sel"][0, :n].tolist() == want["sel"]
        assert r["parents"][0, :n].tolist() == want["parents"]
        assert r["tokens"][0, :n].tolist() == [100 + c for c in want["sel"]]
        assert r["draft_row"][0, :n].tolist() == [int(rows[0, c]) for c in want["sel"]]
        assert (r["sel"][0, n:] == -1).all() and (r["parents"][0, n:] == -1).all()


def test_path_products_are_exact_products():
    rng = np.random.default_rng(5)
    for _ in range(20):
        par, prob = random_pool(rng, 40)
        for i in range(40):
            assert Fraction(float(oracle.path_value(par, prob, i))) == exact_value(par, prob, i)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_objective(seed):
    """Among all sets of N - 1 non-root candidates, the kept one has the largest sum of
    cumulative probabilities (the expected number of accepted nodes under independent
    acceptances), and it contains the parent of each of its members."""
    rng = np.random.default_rng([17, seed])
    C = int(rng.integers(2, 11))
    par, prob = random_pool(rng, C)
    vals = [exact_value(par, prob, i) for i in range(C)]
    for N in range(1, C + 1):
        r = oracle.tree_select(par[None], prob[None], N)
        n = int(r["n_nodes"][0])
        assert n == N
        kept = [int(c) for c in r["sel"][0, :n]]
        assert kept[0] == 0 and kept == sorted(kept)
        best = max(sum(vals[c] for c in s) for s in itertools.combinations(range(1, C), N - 1))
        assert sum(vals[c] for c in kept[1:]) == best
        ks = set(kept)
        for j, c in enumerate(kept[1:], start=1):
            assert int(par[c]) in ks
            assert kept[int(r["parents"][0, j])] == int(par[c])


def test_ties_go_to_the_lower_index():
    """Every probability 1/2: values halve per depth, and within a depth the lowest indices win."""
    par = np.array([[-1, 0, 0, 0, 1, 2, 3, 1]], dtype=np.int32)
    prob = np.full((1, 8), 0.5, dtype=np.float32)
    r = oracle.tree_select(par, prob, 5)
    assert r["sel"][0, :5].tolist() == [0, 1, 2, 3, 4]
    r = oracle.tree_select(par, prob, 6)
    assert r["sel"][0, :6].tolist() == [0, 1, 2, 3, 4, 5]


def test_identity_chain_and_nesting():
    rng = np.random.default_rng(9)
    par, prob = random_pool(rng, 30)
    r = oracle.tree_select(par[None], prob[None], 64)
    assert int(r["n_nodes"][0]) == 30
    assert r["sel"][0, :30].tolist() == list(range(30))
    assert r["parents"][0, :30].tolist() == par.tolist()
    # a chain keeps its first N nodes, whatever the probabilities
    chain = np.arange(-1, 29, dtype=np.int32)
    for N in (1, 5, 30):
        r = oracle.tree_select(chain[None], prob[None], N)
        assert r["sel"][0, :N].tolist() == list(range(N))
    # the tree kept for N is contained in the tree kept for N + 1
    prev = {0}
    for N in range(1, 31):
        kept = set(oracle.tree_select(par[None], prob[None], N)["sel"][0, :N].tolist())
        assert prev <= kept and len(kept) == N
        prev = kept


def test_ragged_and_empty():
    rng = np.random.default_rng(3)
    par, prob = random_pool(rng, 20)
    pars = np.stack([par, par, par])
    probs = np.stack([prob, prob, prob])
    r = oracle.tree_select(pars, probs, 8, n_cand=np.array([20, 5, 0]))
    assert r["n_nodes"].tolist() == [8, 5, 0]
    assert r["sel"][1, :5].tolist() == list(range(5))
    assert (r["sel"][2] == -1).all()
    full = oracle.tree_select(par[None, :5], prob[None, :5], 8)
    assert r["sel"][1].tolist() == full["sel"][0].tolist()


def test_errors():
    par = np.array([[-1, 0, 0, 1]], dtype=np.int32)
    prob = np.array([[0.0, 0.5, 0.5, 0.5]], dtype=np.float32)

    def err(p, q, n=None):
        r = oracle.tree_select(np.array([p], dtype=np.int32), np.array([q], dtype=np.float32), 3,
                               n_cand=None if n is None else np.array([n]))
        if r["err"][0]:
            assert int(r["n_nodes"][0]) == 0 and (r["sel"] == -1).all()
        return oracle.decode_err(r["err"][0])

    assert err(par[0], prob[0]) == (0, 0)
    assert err([0, 0, 0, 1], prob[0]) == (0, oracle.ERR_ROOT)
    assert err([-1, 0, 2, 1], prob[0]) == (2, oracle.ERR_PARENT)
    assert err([-1, 0, 0, 1], [0.0, 0.5, 1.5, 0.5]) == (2, oracle.ERR_PROB)
    assert err([-1, 0, 0, 1], [0.0, 0.5, -0.25, 0.5]) == (2, oracle.ERR_PROB)
    assert err([-1, 0, 0, 1], [0.0, 0.5, 0.5, np.nan]) == (3, oracle.ERR_PROB)
    assert err([-1, 0, 0, 1], [7.0, 0.5, 0.5, 0.5]) == (0, 0)          # the root's entry is unused
    assert err([-1, 0, 0, 5], [0.0, 0.5, 0.5, 0.5], n=3) == (0, 0)     # beyond n_cand: not read
    assert err([-1, 0, 5, 1], [0.0, 0.5, 2.0, 0.5]) == (2, oracle.ERR_PARENT)   # lower code first
    assert err(par[0], prob[0], n=5) == (0, oracle.ERR_NNODES)
    assert err(par[0], prob[0], n=-1) == (0, oracle.ERR_NNODES)
