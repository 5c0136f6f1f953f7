"""Oracle: tree attention as dense masked softmax attention (test infrastructure only).

[MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる" and [GUIDE] section
"Tree Attention：候補を木構造で探索する": every tree node's query attends to the shared
committed prefix and to its own ancestors only, so one forward pass scores every candidate
path.  [GUIDE] section "並列検証：ターゲットモデルの1回のforward passで一括確認する" adds
that the KV cache is what lets all positions be scored in parallel.  What that computes
is ordinary masked softmax attention; this module writes exactly that, one query row at a
time, in float64.

Readings taken where the pages are silent (shapes follow the Llama-3.1-8B draft-head
configuration printed in [GUIDE] section "ドラフトヘッドの構成と学習手順": 32 query heads,
8 key/value heads):
  * scale = 1/sqrt(head_dim) unless given; query head h reads key/value head h // G with
    G = Hq / Hkv (contiguous groups).
  * Node j's key and value sit in cache slot prefix_len + j; queries and keys arrive with
    rotary embedding already applied by the caller.
  * Row i (node i < n_nodes) sees slots [0, prefix_len) and slots prefix_len + j for every
    j with dense[i, j] set.  A row that sees no slot outputs zeros and lse = -inf; padding
    rows are zero as well.
  * A sequence whose sizes do not fit (bad node count, negative prefix, or prefix + nodes
    beyond the cache) gets an error word and all-zero output.
"""

import numpy as np

from .errors import ERR_NNODES, ERR_PREFIX, encode_err


def tree_attention_row(q_row, k_seq, v_seq, prefix, visible_nodes, scale):
    """One query row.  q_row [d]; k_seq, v_seq [S_max, d] of the row's KV head;
    ``visible_nodes`` lists the tree nodes j this row may see.  Returns (out [d], lse)."""
    slots = list(range(int(prefix))) + [int(prefix) + int(j) for j in visible_nodes]
    if not slots:
        return np.zeros(q_row.shape[-1]), -np.inf
    keys = np.asarray(k_seq)[slots].astype(np.float64)
    vals = np.asarray(v_seq)[slots].astype(np.float64)
    scores = scale * (keys @ np.asarray(q_row, dtype=np.float64))
    m = scores.max()
    w = np.exp(scores - m)
    z = w.sum()
    return (w @ vals) / z, m + np.log(z)


def tree_attention(q, k_cache, v_cache, prefix_len, dense, n_nodes=None, scale=None):
    """q [B, N, Hq, d]; k_cache, v_cache [B, Hkv, S_max, d]; prefix_len [B];
    dense bool [B, N, N] from :func:`oracle.tree_build`; n_nodes [B] (default N).

    Returns dict(out float64 [B, N, Hq, d], lse float64 [B, N, Hq], err int32 [B])."""
    q = np.asarray(q)
    B, N, Hq, d = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_nodes = np.full(B, N, dtype=np.int64) if n_nodes is None else np.asarray(n_nodes, np.int64)
    out = np.zeros((B, N, Hq, d), dtype=np.float64)
    lse = np.full((B, N, Hq), -np.inf, dtype=np.float64)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n, P = int(n_nodes[b]), int(prefix_len[b])
        if not 0 <= n <= N:
            err[b] = encode_err(0, ERR_NNODES)
            continue
        if P < 0 or P + n > S_max:
            err[b] = encode_err(0, ERR_PREFIX)
            continue
        for i in range(n):
            visible = [j for j in range(n) if dense[b, i, j]]
            for h in range(Hq):
                g = h // G
                out[b, i, h], lse[b, i, h] = tree_attention_row(
                    q[b, i, h], k_cache[b, g], v_cache[b, g], P, visible, scale)
    return {"out": out, "lse": lse, "err": err}
