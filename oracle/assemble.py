"""Oracle: candidate tree assembly from per-head top-k (test infrastructure only).

[GLOSSARY] section "ツリー構造の候補構築": the candidate tree is the combination of each
head's top candidates (its example: top-3 of head 0, top-3 of head 1 and top-2 of head 2 give
at most 3 x 3 x 2 = 18 paths), laid out on a predefined topology ("Medusa Tree").

Readings taken where the pages are silent:
  * The topology is a parent array shared by the batch (a predefined tree); node numbering
    is topological with node 0 the root.
  * The r-th child of a node (r counted in node order from 0) at depth delta takes the
    rank-r candidate of head delta - 1: tokens[b, i] = topk_idx[b, depth(i) - 1, rank(i)].
  * Node i is verified against draft row depth(i) - 1 (the head that proposed it);
    the root keeps its caller-given token (or -1) and draft row -1.
  * A node deeper than the number of heads, or a rank beyond k, is an error (ERR_RANK).
"""

import numpy as np

from .errors import ERR_ROOT, ERR_PARENT, ERR_RANK, encode_err


def tree_assemble(topk_idx, parents, root_tokens=None):
    """topk_idx int [B, H, k]; parents int [N] (shared topology); root_tokens [B] or None.

    Returns dict(tokens int32 [B, N], draft_row int32 [B, N], err int32 [B])."""
    topk_idx = np.asarray(topk_idx)
    B, H, k = topk_idx.shape
    parents = [int(p) for p in parents]
    N = len(parents)
    tokens = np.full((B, N), -1, dtype=np.int32)
    draft_row = np.full((B, N), -1, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)

    problems = []
    depth = [0] * N
    rank = [0] * N
    if N > 0 and parents[0] != -1:
        problems.append((0, ERR_ROOT))
    for i in range(1, N):
        p = parents[i]
        if not 0 <= p < i:
            problems.append((i, ERR_PARENT))
            continue
        steps, j = 0, i
        while j > 0 and 0 <= parents[j] < j:
            j, steps = parents[j], steps + 1
        depth[i] = steps
        rank[i] = sum(1 for j in range(1, i) if parents[j] == p)
        if depth[i] > H or rank[i] >= k:
            problems.append((i, ERR_RANK))
    if problems:
        err[:] = encode_err(*min(problems))
        return {"tokens": tokens, "draft_row": draft_row, "err": err}

    for b in range(B):
        tokens[b, 0] = -1 if root_tokens is None else int(root_tokens[b])
        for i in range(1, N):
            tokens[b, i] = topk_idx[b, depth[i] - 1, rank[i]]
            draft_row[b, i] = depth[i] - 1
    return {"tokens": tokens, "draft_row": draft_row, "err": err}
