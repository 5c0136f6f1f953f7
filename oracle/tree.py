"""Oracle: candidate tree -> ancestor mask, depths, positions (test infrastructure only).

[MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる" (with its chain-versus-tree
figure) and [GUIDE] section "Tree Attention：候補を木構造で探索する" (with its worked tree
figure) state the rule: each node of the candidate tree may look only at its ancestors,
so that all root-to-leaf candidate paths ride through one batched forward pass.  [GLOSSARY]
section "デプロイと運用上の考慮事項" adds that batched requests each carry their own tree,
which needs padding and mask bookkeeping; ``n_nodes`` is that padding.

Readings taken where the pages are silent:
  * Nodes are numbered topologically: node 0 is the root and ``parents[i] < i``.  This is
    the breadth-first numbering of both tree figures.
  * A node attends to itself as well as its ancestors (its own key/value is part of the
    batched sequence, exactly as in causal decoding).
  * depth(root) = 0; the caller's rotary position of node i is ``prefix_len + depth(i)``.
  * Padding rows (i >= n_nodes) and every row of a sequence with an error get an empty
    mask, depth -1 and position -1.
"""

import numpy as np

from .errors import ERR_ROOT, ERR_PARENT, ERR_DEPTH, ERR_NNODES, ERR_PREFIX, encode_err


def pack_mask(dense):
    """Pack a boolean [..., N, N] ancestor matrix into uint64 words [..., N, ceil(N/64)]:
    bit (j % 64) of word (j // 64) in row i is set iff node j is visible from node i."""
    dense = np.asarray(dense, dtype=bool)
    n = dense.shape[-1]
    words = (n + 63) // 64
    out = np.zeros(dense.shape[:-1] + (words,), dtype=np.uint64)
    for j in range(n):
        bit = np.uint64(1) << np.uint64(j % 64)
        out[..., j // 64] |= np.where(dense[..., j], bit, np.uint64(0))
    return out


def unpack_mask(words, n):
    """Inverse of :func:`pack_mask` for the first ``n`` columns."""
    words = np.asarray(words, dtype=np.uint64)
    dense = np.zeros(words.shape[:-1] + (n,), dtype=bool)
    for j in range(n):
        bit = np.uint64(1) << np.uint64(j % 64)
        dense[..., j] = (words[..., j // 64] & bit) != 0
    return dense


def tree_build(parents, n_nodes=None, depths_in=None, prefix_len=None):
    """Brute-force ancestor walks for a batch of candidate trees.

    parents    int [B, N]   parent of each node, -1 for the root (node 0)
    n_nodes    int [B]      valid nodes per sequence (default N); rows beyond are padding
    depths_in  int [B, N]   optional depths to validate against the walks
    prefix_len int [B]      committed prefix length (default 0), for positions

    Returns a dict with
      ``dense``     bool   [B, N, N]   dense[b, i, j] = j is an ancestor of i, or j == i
      ``mask``      uint64 [B, N, W]   the same, packed by :func:`pack_mask`
      ``depths``    int32  [B, N]      number of proper ancestors
      ``positions`` int32  [B, N]      prefix_len + depth
      ``err``       int32  [B]         error word (see ``oracle.errors``)
    """
    parents = np.asarray(parents, dtype=np.int64)
    B, N = parents.shape
    n_nodes = np.full(B, N, dtype=np.int64) if n_nodes is None else np.asarray(n_nodes, np.int64)
    prefix_len = np.zeros(B, dtype=np.int64) if prefix_len is None else np.asarray(prefix_len, np.int64)
    dense = np.zeros((B, N, N), dtype=bool)
    depths = np.full((B, N), -1, dtype=np.int32)
    positions = np.full((B, N), -1, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)

    for b in range(B):
        n = int(n_nodes[b])
        if not 0 <= n <= N:
            err[b] = encode_err(0, ERR_NNODES)
            continue
        if prefix_len[b] < 0:
            err[b] = encode_err(0, ERR_PREFIX)
            continue
        # Scan nodes in order; the first node with a problem is reported.  Node i is only
        # reached when every earlier node passed, so its parent chain is sound.
        for i in range(n):
            p = int(parents[b, i])
            if i == 0 and p != -1:
                err[b] = encode_err(0, ERR_ROOT)
                break
            if i > 0 and not 0 <= p < i:
                err[b] = encode_err(i, ERR_PARENT)
                break
            # Walk from i to the root, marking every node met (i itself included).
            j, steps = i, 0
            while j != -1:
                dense[b, i, j] = True
                j = int(parents[b, j])
                steps += 1
                if steps > N:
                    raise AssertionError("ancestor walk did not reach the root")
            depths[b, i] = int(dense[b, i].sum()) - 1
            if depths_in is not None and int(depths_in[b, i]) != depths[b, i]:
                err[b] = encode_err(i, ERR_DEPTH)
                break
        if err[b] != 0:
            dense[b] = False
            depths[b] = -1
            continue
        positions[b, :n] = prefix_len[b] + depths[b, :n]

    return {"dense": dense, "mask": pack_mask(dense), "depths": depths,
            "positions": positions, "err": err}
