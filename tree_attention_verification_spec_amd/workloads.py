"""Seeded synthetic inputs for the tree-verification step.

This module only draws inputs: it holds none of the method's arithmetic (no masks, no
attention, no acceptance).  Tests, the benchmark and the smoke check feed the same arrays to
the HIP library and to the CPU oracle.

Shapes follow the pages: Llama-3.1-8B-class grouped-query attention (32 query / 8 key-value
heads, head_dim 128, vocabulary 128256, draft vocabulary 32000 - the draft-head configuration
in "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド", section
"ドラフトヘッドの構成と学習手順"), the 63/127/255-node Medusa tree sizes of
"Medusa（マルチヘッド投機的デコーディング）", section "ツリー構造の候補構築", and draft widths
up to top-8.  No dataset or trained weight is used: every tensor is a seeded random draw.

Seeding: ``numpy.random.default_rng([seed, stream, b])`` with one stream per quantity, so a
quantity of sequence b is the same whatever else is drawn.  Draws are fp32; tensors of a bf16
workload are rounded to bf16 (round to nearest even) and kept as fp32 arrays holding exactly
representable values.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

S_TREE, S_PREFIX, S_Q, S_K, S_V, S_LOGITS, S_NOISE, S_UNIF, S_D2T, S_H, S_WRES, S_WLM, S_TRIALS = range(13)


def rng(seed, stream, b=0):
    return np.random.default_rng([int(seed), int(stream), int(b)])


def round_bf16(x):
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``tree`` is ("random", max_depth) - node i >= 1 hangs under a
    uniformly drawn earlier node of depth < max_depth, per sequence - or ("bfs", caps) - a
    width-first fill where a node at depth t gets caps[t] children, stopped at N nodes and
    shared by the batch."""
    name: str
    seed: int
    B: int
    N: int
    Hq: int
    Hkv: int
    d: int
    prefix: Tuple                      # ("fixed", P) or ("uniform", lo, hi)
    tree: Tuple
    V: int
    sigma_logits: float
    dtype: str                         # "f32" or "bf16"
    modes: Tuple[str, ...]
    draft_rows: str = "per_parent"     # "per_parent" (EAGLE-style) or "per_depth" (Medusa)
    Vd: Optional[int] = None           # draft vocabulary (None: same as V)
    heads: Optional[dict] = None       # {"H", "Dm", "k"} when drafts come from Medusa heads
    n_nodes_range: Optional[Tuple[int, int]] = None   # ragged valid-node counts (padding test)
    extra_slots: int = 0               # cache slots beyond prefix + N

    @property
    def G(self):
        return self.Hq // self.Hkv


CONFIGS = {
    1: Workload("tiny-fp32 B1 4q/1kv d64 P256 tree10 V2048", 1, 1, 10, 4, 1, 64, ("fixed", 256),
                ("bfs", (3, 2)), 2048, 2.0, "f32", ("greedy", "reject"), draft_rows="per_depth"),
    2: Workload("llama3-8b-gqa B1 P2048 tree63 V128256", 2, 1, 63, 32, 8, 128, ("fixed", 2048),
                ("random", 4), 128256, 3.0, "bf16", ("typical", "reject")),
    3: Workload("llama3-8b-gqa B16 P~U[1024,4096] tree127 V128256", 3, 16, 127, 32, 8, 128,
                ("uniform", 1024, 4096), ("random", 5), 128256, 3.0, "bf16", ("reject",)),
    4: Workload("llama3-8b-gqa B4 P8192 tree255 V128256 Vd32000", 4, 4, 255, 32, 8, 128,
                ("fixed", 8192), ("bfs", (8, 6, 4, 3, 2, 2)), 128256, 3.0, "bf16", ("reject",),
                Vd=32000),
    5: Workload("medusa4-heads+llama3-8b-gqa B8 P32768 tree127 V32000", 5, 8, 127, 32, 8, 128,
                ("fixed", 32768), ("bfs", (8, 4, 2, 2)), 32000, 3.0, "bf16", ("reject",),
                draft_rows="per_depth", heads={"H": 4, "Dm": 4096, "k": 8}),
}


def config(i):
    return CONFIGS[int(i)]


def custom(**kw):
    """A workload for tests: defaults are a small bf16 case, override any field."""
    base = Workload("custom", 1000, 2, 37, 8, 2, 128, ("uniform", 60, 333), ("random", 5), 5000,
                    3.0, "bf16", ("greedy", "typical", "reject"))
    return replace(base, **kw)


# ----------------------------------------------------------------------------- trees

def bfs_tree(caps, N):
    parents = [-1]
    depth = [0]
    head = 0
    while len(parents) < N and head < len(parents):
        t = depth[head]
        if t < len(caps):
            for _ in range(caps[t]):
                if len(parents) == N:
                    break
                parents.append(head)
                depth.append(t + 1)
        head += 1
    return np.asarray(parents, dtype=np.int32)


def random_tree(generator, N, max_depth):
    parents = [-1]
    depth = [0]
    for i in range(1, N):
        eligible = [j for j in range(i) if depth[j] < max_depth]
        p = eligible[int(generator.integers(len(eligible)))]
        parents.append(p)
        depth.append(depth[p] + 1)
    return np.asarray(parents, dtype=np.int32)


def trees(w):
    """parents int32 [B, N] and n_nodes int32 [B]."""
    parents = np.zeros((w.B, w.N), dtype=np.int32)
    n_nodes = np.full(w.B, w.N, dtype=np.int32)
    for b in range(w.B):
        g = rng(w.seed, S_TREE, b)
        if w.n_nodes_range is not None:
            n_nodes[b] = int(g.integers(w.n_nodes_range[0], w.n_nodes_range[1] + 1))
        if w.tree[0] == "bfs":
            parents[b] = bfs_tree(w.tree[1], w.N)
        else:
            parents[b] = random_tree(g, w.N, w.tree[1])
    return parents, n_nodes


def prefix_lengths(w):
    if w.prefix[0] == "fixed":
        return np.full(w.B, w.prefix[1], dtype=np.int32)
    lo, hi = w.prefix[1], w.prefix[2]
    return np.asarray([int(rng(w.seed, S_PREFIX, b).integers(lo, hi + 1)) for b in range(w.B)],
                      dtype=np.int32)


def s_max(w):
    hi = w.prefix[1] if w.prefix[0] == "fixed" else w.prefix[2]
    return int(hi) + w.N + w.extra_slots


def _cast(w, x):
    return round_bf16(x) if w.dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------- attention

def attention_inputs(w, poison=False):
    """q [B, N, Hq, d]; k_cache, v_cache [B, Hkv, S_max, d] (node j at slot prefix + j),
    all fp32 arrays (bf16-exact for bf16 workloads).  With ``poison`` the cache slots past
    prefix + n_nodes, and the query rows of padding nodes, are NaN."""
    parents, n_nodes = trees(w)
    P = prefix_lengths(w)
    S = s_max(w)
    q = np.empty((w.B, w.N, w.Hq, w.d), dtype=np.float32)
    k = np.empty((w.B, w.Hkv, S, w.d), dtype=np.float32)
    v = np.empty((w.B, w.Hkv, S, w.d), dtype=np.float32)
    for b in range(w.B):
        q[b] = _cast(w, rng(w.seed, S_Q, b).standard_normal((w.N, w.Hq, w.d), dtype=np.float32))
        k[b] = _cast(w, rng(w.seed, S_K, b).standard_normal((w.Hkv, S, w.d), dtype=np.float32))
        v[b] = _cast(w, rng(w.seed, S_V, b).standard_normal((w.Hkv, S, w.d), dtype=np.float32))
        if poison:
            k[b, :, P[b] + n_nodes[b]:] = np.nan
            v[b, :, P[b] + n_nodes[b]:] = np.nan
            q[b, n_nodes[b]:] = np.nan
    return {"q": q, "k_cache": k, "v_cache": v, "prefix_len": P, "parents": parents,
            "n_nodes": n_nodes, "S_max": S, "scale": 1.0 / np.sqrt(w.d)}


# ----------------------------------------------------------------------------- verify

def d2t_table(w):
    """Draft->target id table (sorted seeded subset) and its inverse (-1 where unmapped)."""
    if w.Vd is None or w.Vd == w.V:
        return None, None
    d2t = np.sort(rng(w.seed, S_D2T).choice(w.V, size=w.Vd, replace=False)).astype(np.int32)
    t2d = np.full(w.V, -1, dtype=np.int32)
    t2d[d2t] = np.arange(w.Vd, dtype=np.int32)
    return d2t, t2d


def target_logits(w, b):
    return (rng(w.seed, S_LOGITS, b).standard_normal((w.N, w.V), dtype=np.float32)
            * np.float32(w.sigma_logits))


def uniforms(w):
    return np.stack([rng(w.seed, S_UNIF, b).random(w.N, dtype=np.float32) for b in range(w.B)])


def _softmax64(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _top(p, k):
    """Indices of the k largest entries, lower index first on ties."""
    return np.argsort(-np.asarray(p), kind="stable")[:k]


def verify_inputs(w, parents=None):
    """Target logits, draft rows and candidate tokens for workloads whose drafts are noisy
    copies of target rows (everything except Medusa-head workloads).

    Draft row of proposing node s: softmax(logits[s] + N(0, 0.5)), over the draft vocabulary
    when there is one.  Per-parent rows: s is the parent; per-depth rows: s is the first node
    of the previous depth.  The children of a node take the top candidates of their row in
    sibling order (mapped to target ids through d2t)."""
    if parents is None:
        parents, _ = trees(w)
    d2t, t2d = d2t_table(w)
    Vd = w.V if d2t is None else w.Vd
    B, N = w.B, w.N
    logits = np.empty((B, N, w.V), dtype=np.float32)
    tokens = np.full((B, N), -1, dtype=np.int32)
    draft_row = np.full((B, N), -1, dtype=np.int32)
    rows_per_seq = []
    for b in range(B):
        logits[b] = target_logits(w, b)
        par = parents[b]
        kids = [[] for _ in range(N)]
        depth = np.zeros(N, dtype=np.int64)
        for c in range(1, N):
            kids[par[c]].append(c)
            depth[c] = depth[par[c]] + 1
        if w.draft_rows == "per_parent":
            sources = [p for p in range(N) if kids[p]]
            row_of_child = {c: sources.index(par[c]) for c in range(1, N)}
        else:
            maxd = int(depth.max())
            sources = [int(np.flatnonzero(depth == t)[0]) for t in range(maxd)]
            row_of_child = {c: int(depth[c]) - 1 for c in range(1, N)}
        rows_per_seq.append(sources)
        for c in range(1, N):
            draft_row[b, c] = row_of_child[c]
    R = max(len(s) for s in rows_per_seq)
    draft = np.zeros((B, R, Vd), dtype=np.float32)
    for b in range(B):
        noise = rng(w.seed, S_NOISE, b).standard_normal((R, Vd), dtype=np.float32) * np.float32(0.5)
        for r, s in enumerate(rows_per_seq[b]):
            src = logits[b, s] if d2t is None else logits[b, s, d2t]
            draft[b, r] = _softmax64(src.astype(np.float64) + noise[r]).astype(np.float32)
        par = parents[b]
        kids = [[] for _ in range(N)]
        for c in range(1, N):
            kids[par[c]].append(c)
        for p in range(N):
            if not kids[p]:
                continue
            r = draft_row[b, kids[p][0]]
            best = _top(draft[b, r], len(kids[p]))
            for rank, c in enumerate(kids[p]):
                tok = int(best[rank % len(best)])      # repeats only when Vd < #children
                tokens[b, c] = tok if d2t is None else int(d2t[tok])
    return {"target_logits": logits, "draft_probs": draft, "draft_row": draft_row,
            "tokens": tokens, "uniforms": uniforms(w), "t2d": t2d, "d2t": d2t, "R": R, "Vd": Vd}


# ----------------------------------------------------------------------------- heads

def heads_inputs(w):
    """h [B, Dm] ~ N(0, 1); W_res [H, Dm, Dm] and W_lm [V, Dm] ~ N(0, 0.02); all bf16."""
    H, Dm = w.heads["H"], w.heads["Dm"]
    h = round_bf16(rng(w.seed, S_H).standard_normal((w.B, Dm), dtype=np.float32))
    W_res = np.empty((H, Dm, Dm), dtype=np.float32)
    for j in range(H):
        W_res[j] = round_bf16(rng(w.seed, S_WRES, j).standard_normal((Dm, Dm), dtype=np.float32)
                              * np.float32(0.02))
    W_lm = round_bf16(rng(w.seed, S_WLM).standard_normal((w.V, Dm), dtype=np.float32)
                      * np.float32(0.02))
    return {"h": h, "W_res": W_res, "W_lm": W_lm, "k": w.heads["k"]}


def heads_target_inputs(w):
    """Target logits and uniforms for a Medusa-head workload (drafts come from the heads)."""
    logits = np.stack([target_logits(w, b) for b in range(w.B)])
    return {"target_logits": logits, "uniforms": uniforms(w)}


# ----------------------------------------------------------------------------- tree selection

def select_inputs(w, vi=None, parents=None):
    """A candidate pool from a workload's tree: parents, tokens and draft rows as drafted, and
    each candidate's draft probability looked up in its draft row (through the target->draft
    map when the drafter has its own vocabulary).  The root's entry is 1."""
    if parents is None:
        parents, _ = trees(w)
    if vi is None:
        vi = verify_inputs(w, parents)
    B, N = w.B, w.N
    prob = np.ones((B, N), dtype=np.float32)
    for b in range(B):
        for c in range(1, N):
            tok = int(vi["tokens"][b, c])
            x = tok if vi["t2d"] is None else int(vi["t2d"][tok])
            prob[b, c] = vi["draft_probs"][b, vi["draft_row"][b, c], x]
    return {"cand_parents": np.asarray(parents, dtype=np.int32), "cand_prob": prob,
            "cand_tokens": vi["tokens"], "cand_row": vi["draft_row"]}


def random_pool(seed, B, C, max_depth=8, power=2.0):
    """Seeded random candidate pools: candidate i attaches to a uniform earlier candidate of depth
    < max_depth; probabilities U(0,1)^power as float32 (skewed towards small values, as the
    draft probabilities of lower-ranked candidates are); tokens and rows are distinct tags."""
    par = np.full((B, C), -1, dtype=np.int32)
    prob = np.ones((B, C), dtype=np.float32)
    for b in range(B):
        g = rng(seed, S_TREE, b)
        depth = np.zeros(C, dtype=np.int64)
        ok = [0]
        for i in range(1, C):
            p = ok[int(g.integers(0, len(ok)))]
            par[b, i] = p
            depth[i] = depth[p] + 1
            if depth[i] < max_depth:
                ok.append(i)
        prob[b, 1:] = (g.random(C - 1) ** power).astype(np.float32)
    tokens = (np.arange(C, dtype=np.int32)[None, :] * 7 + 1000 * np.arange(B, dtype=np.int32)[:, None])
    rows = np.maximum(par, 0).astype(np.int32)
    return {"cand_parents": par, "cand_prob": prob, "cand_tokens": tokens.astype(np.int32), "cand_row": rows}


# ----------------------------------------------------------------------------- target LM head

def lm_head_inputs(seed, B, N, Dm, V, parents=None, max_depth=4):
    """The target's last hidden states at the tree nodes, h ~ N(0, 1), and its LM head
    W ~ N(0, 0.02) [V, Dm], both rounded to bf16 (fp32 arrays holding bf16 values); a tree per
    sequence (node i attaches to a uniform earlier node of depth < max_depth, unless given) and
    uniform candidate tokens."""
    h = round_bf16(np.stack([rng(seed, S_H, b).standard_normal((N, Dm), dtype=np.float32) for b in range(B)]))
    W = round_bf16(rng(seed, S_WLM).standard_normal((V, Dm), dtype=np.float32) * np.float32(0.02))
    if parents is None:
        parents = np.stack([random_tree(rng(seed, S_TREE, b), N, max_depth) for b in range(B)]).astype(np.int32)
    tokens = np.stack([rng(seed, S_LOGITS, b).integers(0, V, size=N) for b in range(B)]).astype(np.int32)
    tokens[:, 0] = -1
    return {"hidden": h, "W": W, "parents": np.asarray(parents, dtype=np.int32), "tokens": tokens}
