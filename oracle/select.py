"""Oracle: dynamic candidate-tree selection by cumulative draft probability (test infrastructure only).

[MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる": a wider and deeper tree raises the
expected accepted length but costs verification work, and EAGLE-2's dynamic tree shapes the
tree by how confident the context is, balancing the two.  [GLOSSARY] section "EAGLE: Medusaの
発展形" and [GUIDE] section "EAGLE-1/2からの進化" name the same idea (a context-aware draft
tree whose topology is chosen per input).  The pages give no formula; this module takes the
plainest reading consistent with them:

  * The drafter proposes a candidate tree (parents in topological order, node 0 the root) and
    the probability p_i its draft distribution gave each candidate's token.
  * A candidate's value is its cumulative draft probability: the product of p along its path
    from the root (the root's own entry is ignored; its value is 1).  Under independent
    acceptances the expected accepted length of a tree is the sum of these values over its
    non-root nodes, so the best tree of a given size keeps the largest values.
  * The root and the N - 1 non-root candidates of largest value are kept (ties: lower candidate
    index first).  Because every p lies in [0, 1], a child's value never exceeds its parent's,
    and the parent has the lower index, so the kept set always contains the parents of its
    members: it is itself a tree.
  * Kept candidates stay in candidate order, which keeps the numbering topological; parents
    are renumbered, tokens and draft rows are carried along (draft rows keep indexing the
    drafter's rows).

Precision: the values decide an integer result, so both this oracle and the GPU take that
decision in the same arithmetic: float64 products of the float32 probabilities, multiplied
from the root downwards, each product rounded once (IEEE round to nearest).  Two candidates
whose values compare equal are ordered by index.

Errors (smallest word wins, as for the other steps): n_cand outside [0, C] (ERR_NNODES at node
0), parents[0] != -1 (ERR_ROOT), parents[i] outside [0, i) (ERR_PARENT), p_i not a number in
[0, 1] for a non-root candidate (ERR_PROB).  A sequence with an error keeps nothing
(n_nodes 0, every output -1).
"""

import numpy as np

from .errors import ERR_ROOT, ERR_PARENT, ERR_NNODES, ERR_PROB, encode_err


def path_value(parents, prob, i):
    """Cumulative draft probability of candidate i: float64 product of prob along the path,
    root first (the root contributes nothing)."""
    path = []
    j = i
    while j > 0:
        path.append(j)
        j = int(parents[j])
    v = np.float64(1.0)
    for j in reversed(path):
        v = np.float64(v * np.float64(np.float32(prob[j])))
    return v


def tree_select(cand_parents, cand_prob, N, n_cand=None, cand_tokens=None, cand_row=None):
    """Keep the best N-node subtree of each sequence's candidate tree.

    cand_parents int [B, C]    parent of each candidate, -1 for the root (candidate 0)
    cand_prob    f32 [B, C]    draft probability of each candidate's token (root entry unused)
    N            int           node capacity of the output tree (>= 1)
    n_cand       int [B]       valid candidates per sequence (default C)
    cand_tokens  int [B, C]    optional, carried to the kept nodes
    cand_row     int [B, C]    optional draft-row index of each candidate, carried along

    Returns dict with ``sel`` int32 [B, N] (candidate index of kept node j, -1 past n_nodes),
    ``parents`` int32 [B, N], ``tokens`` int32 [B, N], ``draft_row`` int32 [B, N],
    ``n_nodes`` int32 [B], ``err`` int32 [B] and ``value`` float64 [B, N] (the kept nodes'
    cumulative probabilities, NaN past n_nodes)."""
    cand_parents = np.asarray(cand_parents)
    cand_prob = np.asarray(cand_prob, dtype=np.float32)
    B, C = cand_parents.shape
    if n_cand is None:
        n_cand = np.full(B, C, dtype=np.int64)
    out = {k: np.full((B, N), -1, dtype=np.int32) for k in ("sel", "parents", "tokens", "draft_row")}
    out["n_nodes"] = np.zeros(B, dtype=np.int32)
    out["err"] = np.zeros(B, dtype=np.int32)
    out["value"] = np.full((B, N), np.nan)
    for b in range(B):
        n = int(n_cand[b])
        if not 0 <= n <= C:
            out["err"][b] = encode_err(0, ERR_NNODES)
            continue
        par = [int(x) for x in cand_parents[b, :n]]
        problems = []
        if n > 0 and par[0] != -1:
            problems.append((0, ERR_ROOT))
        for i in range(1, n):
            if not 0 <= par[i] < i:
                problems.append((i, ERR_PARENT))
            p = float(cand_prob[b, i])
            if not (0.0 <= p <= 1.0):        # also rejects NaN
                problems.append((i, ERR_PROB))
        if problems:
            out["err"][b] = encode_err(*min(problems))
            continue
        if n == 0:
            continue
        value = [path_value(par, cand_prob[b], i) for i in range(n)]
        ranked = sorted(range(1, n), key=lambda i: (-value[i], i))
        keep = sorted([0] + ranked[:N - 1])
        new_index = {c: j for j, c in enumerate(keep)}
        for j, c in enumerate(keep):
            out["sel"][b, j] = c
            out["parents"][b, j] = -1 if c == 0 else new_index[par[c]]
            if cand_tokens is not None:
                out["tokens"][b, j] = int(cand_tokens[b, c])
            if cand_row is not None:
                out["draft_row"][b, j] = int(cand_row[b, c])
            out["value"][b, j] = value[c]
        out["n_nodes"][b] = len(keep)
    return out
