"""Oracle: per-node acceptance, longest accepted path and bonus token (test infrastructure only).

What the pages fix:
  * [GUIDE] section "棄却サンプリング：出力品質を保証する": a drafted token x is accepted
    with probability min(1, T[x] / D[x]) (T the target distribution, D the draft's); on a
    rejection a replacement is drawn from the residual norm(relu(T - D)); this keeps the
    output distribution equal to the target's.  The note in the same section: once a
    candidate is rejected, every candidate after it is dropped.
  * [GLOSSARY] section "Medusa-1とMedusa-2の違い": typical acceptance keeps a candidate
    x_i when the target probability p(x_i) is at least an entropy-dependent threshold; it is
    an approximation of the target distribution.
  * [MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる": one pass scores all
    paths of the tree and the path that passes acceptance the longest is kept.
  * [GUIDE] section "結論・成果" quotes its speedups at temperature 0.

Readings taken where the pages are silent or loose:
  * T_p, the distribution of the children of node p, is the softmax of node p's target
    logits row.  Node c (parent p, token x, draft row r = draft_row[c]) is tested on T_p.
  * GREEDY (temperature 0): T_p collapses onto argmax T_p (lowest token id on ties), so c
    is accepted iff x is that argmax; the bonus token is the argmax of the final row.
  * TYPICAL: threshold tau_p = min(eps, delta * exp(-H_p)) with H_p the entropy of T_p in
    nats (the threshold form of the Medusa paper the glossary cites); delta = +inf gives a
    fixed threshold eps.  Accept iff T_p[x] >= tau_p.  The bonus token is sampled from the
    final row's T.
  * REJECT: accept iff u_c * D[x] < T_p[x], the same event as u_c < min(1, T_p[x]/D[x]) for
    D[x] > 0 (for D[x] = 0 the candidate is accepted iff T_p[x] > 0).  The nodes are tested
    independently (one uniform each) and combined by the rules below.
  * A node survives iff it and every ancestor below the root were accepted.  The kept node
    m is the surviving node of greatest depth, smallest index on ties; accept_len is its
    depth and path lists the nodes root..m.
  * Bonus in REJECT mode: if m has children, draw from norm(relu(T_m - D)) with D the draft
    row of m's lowest-index child (all children of m share a row in both Medusa per-depth
    and EAGLE per-parent layouts); if that residual sums to zero, or m has no child, draw
    from T_m.
  * Draws use uniforms[b, 0] and inverse-CDF sampling: the smallest token t whose running
    sum of q from token 0 upward exceeds u * Z, Z the total sum, both accumulated in float64
    in ascending token order.
  * WALK (the tree-lossless variant of REJECT): the tree is walked from the root.  At node p
    the children are tried in index order against a running distribution R, first R = T_p;
    child c (token x, uniform u_c, draft row D) is accepted iff u_c * D[x] < R[x]; on a
    rejection R becomes norm(relu(R - D)) before the next sibling is tried, which is the
    guide's residual rule applied once per rejected sibling, so every sibling is a fresh
    draw against what the earlier rejections left.  The first accepted child becomes the new
    p; when every child of p is rejected, or p has none, the walk stops at m = p and the
    bonus is drawn from R (from T_m when m has no child, or when R has summed to zero, after
    which every later sibling counts as rejected).  With children drawn i.i.d. from D this
    keeps the law of the emitted tokens equal to the target's on any tree (the residual
    argument applied sibling after sibling); REJECT is exact only on chains.  The children of
    one node must share a draft row (as in both layouts above): a child whose row differs
    from its first sibling's is ERR_DRAFTROW.  node_accept marks the walk's path.
  * Draft rows may live on a smaller draft vocabulary: t2d[x] maps target token x to a
    draft index, -1 for tokens the draft cannot emit (their draft probability is 0).  A
    candidate whose entry lies outside [-1, Vd) is an error; any other such entry is read
    as -1.
"""

import numpy as np

from .errors import (ERR_ROOT, ERR_PARENT, ERR_DEPTH, ERR_NNODES, ERR_TOKEN, ERR_DRAFTROW,
                     ERR_NONFINITE, ERR_MAP, encode_err)

MODE_GREEDY = 0
MODE_TYPICAL = 1
MODE_REJECT = 2
MODE_WALK = 3


def sample_inverse_cdf(q, u):
    """Smallest index t with sum(q[0..t]) > u * sum(q), sums in float64 from index 0 upward.

    Returns (t, margin) where margin is the distance, relative to the total, between u * Z
    and the nearer of the two cumulative sums around it."""
    q = [float(v) for v in np.asarray(q, dtype=np.float64)]
    z = 0.0
    for v in q:
        z += v
    thr = float(u) * z
    c_prev, c = 0.0, 0.0
    for t, v in enumerate(q):
        c_prev, c = c, c + v
        if c > thr:
            return t, min(c - thr, thr - c_prev) / z
    return len(q) - 1, 0.0


def _row_stats(row):
    """max, lowest-index argmax, softmax T (float64) and its entropy in nats."""
    row = np.asarray(row, dtype=np.float64)
    mx = row.max()
    argmax = int(np.flatnonzero(row == mx)[0])
    e = np.exp(row - mx)
    T = e / e.sum()
    pos = T > 0
    H = float(-(T[pos] * np.log(T[pos])).sum())
    # Greedy margin: gap from the top logit to the best other logit.
    others = np.delete(row, argmax)
    gap = float(mx - others.max()) if others.size else np.inf
    return {"max": mx, "argmax": argmax, "T": T, "H": H, "gap": gap}


def _draft_on_target_vocab(draft_row_probs, t2d, V):
    """The draft row as a distribution over target token ids."""
    d = np.asarray(draft_row_probs, dtype=np.float64)
    if t2d is None:
        return d[:V].copy()
    out = np.zeros(V, dtype=np.float64)
    for v in range(V):
        if 0 <= t2d[v] < len(d):
            out[v] = d[t2d[v]]
    return out


def _residual_step(Rv, D):
    """One rejected sibling: (norm(relu(R - D)), its normaliser); None for a zero residual."""
    Rn = np.maximum(Rv - D, 0.0)
    z = float(Rn.sum())
    return (Rn / z if z > 0 else None), z


def residual_after_rejections(T, D, j):
    """The running distribution after j rejected siblings that share draft row D: R_0 = T and
    R_i = norm(relu(R_(i-1) - D)); None once a residual has summed to zero."""
    Rv = np.asarray(T, dtype=np.float64).copy()
    D = np.asarray(D, dtype=np.float64)
    for _ in range(j):
        Rv, _ = _residual_step(Rv, D)
        if Rv is None:
            return None
    return Rv


def _walk(b, n, children, stats, logits, tokens, uniforms, draft_probs, draft_row, t2d, V, margin):
    """WALK mode for one sequence (see the module's readings).  Returns the path root..m and
    the distribution of the bonus draw (None: T_m).  Fills margin[b, c] for every tested
    child with the distance of its test from the boundary, relative to the magnitudes that
    enter it: writing R = relu(T - c D) / s (c, s follow from the normalisers of the earlier
    rejections), |u D[x] s - (T[x] - c D[x])| / (T[x] + c D[x] + u D[x] s)."""
    cur, chain = 0, [0]
    while True:
        kids = children[cur]
        if not kids:
            return chain, None
        T = stats[cur]["T"]
        D = _draft_on_target_vocab(draft_probs[b, int(draft_row[b, kids[0]])], t2d, V)
        Rv = T.copy()
        c_sc, s_sc = 0.0, 1.0
        live, nxt = True, None
        for c in kids:
            x, u = int(tokens[b, c]), float(uniforms[b, c])
            if live:
                if D[x] > 0:
                    num = abs(u * D[x] * s_sc - (T[x] - c_sc * D[x]))
                    margin[b, c] = num / (T[x] + c_sc * D[x] + u * D[x] * s_sc)
                if u * D[x] < Rv[x]:
                    nxt = c
                    break
                Rv, z = _residual_step(Rv, D)
                c_sc, s_sc = c_sc + s_sc, s_sc * z
                live = Rv is not None
        if nxt is None:
            return chain, (Rv if live else None)
        chain.append(nxt)
        cur = nxt


def verify(target_logits, tokens, parents, uniforms, mode, *, draft_probs=None, draft_row=None,
           t2d=None, n_nodes=None, eps=0.09, delta=0.3, max_depth=None):
    """target_logits [B, N, V] (row p = target logits at node p); tokens, parents [B, N];
    uniforms [B, N] (column 0 for the bonus draw, column c for node c); draft_probs
    [B, R, Vd]; draft_row [B, N]; t2d [V] or None (identity, Vd == V); n_nodes [B].

    Returns a dict: accept_len [B], path [B, max_depth+1] (-1 padded), bonus [B],
    node_accept uint8 [B, N] (per-node test result, root 1), err [B], and diagnostics
    m [B], margin [B, N] (distance of each test from its decision boundary, inf where the
    test is exact), bonus_margin [B]."""
    logits = target_logits
    B, N, V = logits.shape
    if max_depth is None:
        max_depth = N - 1
    n_nodes = np.full(B, N, dtype=np.int64) if n_nodes is None else np.asarray(n_nodes, np.int64)
    drafted = mode in (MODE_REJECT, MODE_WALK)
    if drafted:
        R, Vd = draft_probs.shape[1], draft_probs.shape[2]

    accept_len = np.zeros(B, dtype=np.int32)
    path = np.full((B, max_depth + 1), -1, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    node_accept = np.zeros((B, N), dtype=np.uint8)
    err = np.zeros(B, dtype=np.int32)
    m_out = np.full(B, -1, dtype=np.int32)
    margin = np.full((B, N), np.inf)
    bonus_margin = np.full(B, np.inf)

    for b in range(B):
        n = int(n_nodes[b])
        if not 0 <= n <= N:
            err[b] = encode_err(0, ERR_NNODES)
            continue
        if n == 0:
            continue
        par = [int(parents[b, c]) for c in range(n)]

        # Structural checks; depth is found by walking up to the root.
        problems = []
        depth = [0] * n
        if par[0] != -1:
            problems.append((0, ERR_ROOT))
        for c in range(1, n):
            if not 0 <= par[c] < c:
                problems.append((c, ERR_PARENT))
                continue
            j, steps = c, 0
            while j > 0 and 0 <= par[j] < j:
                j, steps = par[j], steps + 1
            depth[c] = steps
            if steps > max_depth:
                problems.append((c, ERR_DEPTH))
            x = int(tokens[b, c])
            if not 0 <= x < V:
                problems.append((c, ERR_TOKEN))
            if drafted:
                if not 0 <= int(draft_row[b, c]) < R:
                    problems.append((c, ERR_DRAFTROW))
                if t2d is not None and 0 <= x < V and not -1 <= int(t2d[x]) < Vd:
                    problems.append((c, ERR_MAP))
        children = {p: [] for p in range(n)}
        for c in range(1, n):
            if 0 <= par[c] < c:
                children[par[c]].append(c)
        internal = [p for p in range(n) if children[p]]
        if mode == MODE_WALK:
            for p in internal:
                r0 = int(draft_row[b, children[p][0]])
                for c in children[p][1:]:
                    if 0 <= r0 < R and 0 <= int(draft_row[b, c]) < R and int(draft_row[b, c]) != r0:
                        problems.append((c, ERR_DRAFTROW))
        for p in internal:
            if not np.all(np.isfinite(logits[b, p])):
                problems.append((p, ERR_NONFINITE))
        if problems:
            err[b] = encode_err(*min(problems))
            continue

        stats = {p: _row_stats(logits[b, p]) for p in internal}

        walk_q = None
        if mode == MODE_WALK:
            chain, walk_q = _walk(b, n, children, stats, logits, tokens, uniforms, draft_probs,
                                  draft_row, t2d, V, margin)
            m = chain[-1]
            accepted = [c in chain for c in range(n)]
        else:
            accepted = [True] * n
        # Per-node tests (the walk tests its nodes as it goes).
        for c in range(1, n if mode != MODE_WALK else 1):
            p, x = par[c], int(tokens[b, c])
            st = stats[p]
            t_px = st["T"][x]
            if mode == MODE_GREEDY:
                accepted[c] = x == st["argmax"]
            elif mode == MODE_TYPICAL:
                tau = min(eps, delta * np.exp(-st["H"]))
                accepted[c] = t_px >= tau
                if t_px > 0 and tau > 0:
                    margin[b, c] = abs(np.log(t_px) - np.log(tau))
            elif mode == MODE_REJECT:
                r = int(draft_row[b, c])
                if t2d is None:
                    d_x = float(draft_probs[b, r, x])
                else:
                    d_x = float(draft_probs[b, r, t2d[x]]) if t2d[x] >= 0 else 0.0
                u = float(uniforms[b, c])
                accepted[c] = u * d_x < t_px
                if d_x > 0:
                    margin[b, c] = abs(u - min(1.0, t_px / d_x))
            else:
                raise ValueError("unknown mode")

        if mode != MODE_WALK:
            # A node survives iff every node on its chain below the root was accepted
            # (candidates after a rejection are dropped).
            survives = [False] * n
            for c in range(n):
                ok, j = True, c
                while j > 0:
                    ok = ok and accepted[j]
                    j = par[j]
                survives[c] = ok

            # Deepest survivor, smallest index on ties.
            m = 0
            for c in range(1, n):
                if survives[c] and depth[c] > depth[m]:
                    m = c
            chain = []
            j = m
            while j != -1:
                chain.append(j)
                j = par[j] if j > 0 else -1
            chain.reverse()

        # Bonus token from row m.
        row_m = logits[b, m]
        if m not in stats and not np.all(np.isfinite(row_m)):
            err[b] = encode_err(m, ERR_NONFINITE)
            continue
        st_m = stats[m] if m in stats else _row_stats(row_m)
        u0 = float(uniforms[b, 0])
        if mode == MODE_GREEDY:
            tok, bm = st_m["argmax"], st_m["gap"]
        elif mode == MODE_TYPICAL:
            tok, bm = sample_inverse_cdf(st_m["T"], u0)
        elif mode == MODE_WALK:
            tok, bm = sample_inverse_cdf(st_m["T"] if walk_q is None else walk_q, u0)
        else:
            q = st_m["T"]
            if children[m]:
                r = int(draft_row[b, min(children[m])])
                d = _draft_on_target_vocab(draft_probs[b, r], t2d, V)
                resid = np.maximum(st_m["T"] - d, 0.0)
                if resid.sum() > 0:
                    q = resid
            tok, bm = sample_inverse_cdf(q, u0)

        accept_len[b] = depth[m]
        path[b, :len(chain)] = chain
        bonus[b] = tok
        node_accept[b, 0] = 1
        for c in range(1, n):
            node_accept[b, c] = 1 if accepted[c] else 0
        m_out[b] = m
        bonus_margin[b] = bm

    return {"accept_len": accept_len, "path": path, "bonus": bonus, "node_accept": node_accept,
            "err": err, "m": m_out, "margin": margin, "bonus_margin": bonus_margin}
