"""Oracle: candidate tree assembly (test infrastructure only): from per-head top-k on a predefined
topology (Medusa), and from per-node draft distributions, each node's children taking the top
candidates of the distribution computed at it (EAGLE style, tree_assemble_rows below).

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

from .errors import ERR_ROOT, ERR_PARENT, ERR_RANK, ERR_NNODES, ERR_DRAFTROW, ERR_NONFINITE, ERR_MAP, encode_err


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


def tree_assemble_rows(draft_probs, parents, draft_row, d2t=None, V=None, n_nodes=None, root_tokens=None):
    """Candidate tokens of a draft tree from per-node draft distributions (EAGLE style).

    [MTP] section "EAGLE：token ではなく「特徴量」を先読みする": the drafter's predicted feature
    goes through the target's LM head, which gives a distribution over candidate tokens; the
    step is repeated to grow a draft tree.  [GUIDE] section "Tree Attention：候補を木構造で探索する":
    several candidates are proposed for one position (its figure: the root has three
    children, t1a has two).  [GUIDE]'s SGLang example sets eagle-topk 8, the number of
    candidates taken per expanded node.

    draft_probs [B, R, Vd] (the draft distributions); parents, draft_row int [B, N];
    d2t [Vd] int or None (draft id -> target id; None: identity, V = Vd); n_nodes [B] or None.

    Readings taken where the pages are silent:
      * The children of node p, in node order c_0 < c_1 < ..., are p's candidates: they share
        the draft row r = draft_row[c_0] (the distribution computed at p), and child c_j takes
        the j-th entry of that row ranked by probability, highest first, ties to the lower
        draft id (-0.0 and 0.0 are equal).  Its token is d2t[id] and its cand_prob D_r[id].
      * The root keeps root_tokens[b] (or -1) and cand_prob 1.
      * Errors (smallest (node, code) wins; sequence-level first): n_nodes outside [0, N]
        (ERR_NNODES at node 0); parents[0] != -1 (ERR_ROOT); parents[c] outside [0, c)
        (ERR_PARENT); draft_row[c] outside [0, R), or differing from its first sibling's
        (ERR_DRAFTROW at c); a child ranked j >= Vd (ERR_RANK at c); a ranked row holding a
        NaN (ERR_NONFINITE at the parent's first child); d2t[id] outside [0, V) (ERR_MAP at c).
        A sequence with an error, and every padding node, gets token -1 and cand_prob NaN.

    Returns dict(tokens int32 [B, N], cand_prob float32 [B, N], err int32 [B])."""
    D = np.asarray(draft_probs)
    B, R, Vd = D.shape
    parents = np.asarray(parents)
    draft_row = np.asarray(draft_row)
    N = parents.shape[1]
    if V is None:
        V = Vd
    if n_nodes is None:
        n_nodes = np.full(B, N, dtype=np.int64)
    tokens = np.full((B, N), -1, dtype=np.int32)
    cand_prob = np.full((B, N), np.nan, dtype=np.float32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if not 0 <= n <= N:
            err[b] = encode_err(0, ERR_NNODES)
            continue
        problems = []
        if n > 0 and int(parents[b, 0]) != -1:
            problems.append((0, ERR_ROOT))
        children = [[] for _ in range(N)]
        for c in range(1, n):
            p = int(parents[b, c])
            if not 0 <= p < c:
                problems.append((c, ERR_PARENT))
            else:
                children[p].append(c)
        picks = {}
        for p in range(n):
            kids = children[p]
            if not kids:
                continue
            r0 = int(draft_row[b, kids[0]])
            ranked = None
            if 0 <= r0 < R:
                row = D[b, r0].astype(np.float64)
                if np.isnan(row).any():
                    problems.append((kids[0], ERR_NONFINITE))
                # probability high to low, then draft id low to high (a sort by two keys, the
                # last one primary; it compares values, so -0.0 and 0.0 are equal)
                ranked = np.lexsort((np.arange(Vd), -row))
            for j, c in enumerate(kids):
                r = int(draft_row[b, c])
                if not 0 <= r < R or r != r0:
                    problems.append((c, ERR_DRAFTROW))
                    continue
                if j >= Vd:
                    problems.append((c, ERR_RANK))
                    continue
                i = ranked[j]
                t = i if d2t is None else int(d2t[i])
                if not 0 <= t < V:
                    problems.append((c, ERR_MAP))
                    continue
                picks[c] = (t, D[b, r, i])
        if problems:
            err[b] = encode_err(*min(problems))
            continue
        if n > 0:
            tokens[b, 0] = -1 if root_tokens is None else int(root_tokens[b])
            cand_prob[b, 0] = 1.0
        for c, (t, pr) in picks.items():
            tokens[b, c] = t
            cand_prob[b, c] = pr
    return {"tokens": tokens, "cand_prob": cand_prob, "err": err}
