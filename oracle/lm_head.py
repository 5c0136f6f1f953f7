"""Oracle: the target model's LM head fused with the row statistics verification reads
(test infrastructure only).

[GUIDE] section "並列検証：ターゲットモデルの1回のforward passで一括確認する": one forward pass of
the target model gives the probability distribution at every candidate position; [MTP] section
"ツリー検証：候補を「木」に束ねて1回で確かめる": all tree nodes ride through that one pass.  The
distribution of node p's children is T_p = softmax(W h_p), W the target's LM head and h_p the
target's last hidden state at node p ([GUIDE] section "ドラフトヘッドの構成と学習手順": hidden
size 4096, vocabulary 128256 for the Llama-3.1-8B-class target).  Verification reads only a few
numbers of each row: its maximum and lowest arg-maximum (greedy acceptance and the greedy bonus),
S = sum exp(l - max) and A = sum exp(l - max) (l - max) (so that T_p[x] = exp(l[x] - max) / S
and the entropy ln S - A / S needed by typical acceptance), and the logit of each child's token
in its parent's row.

Readings taken where the pages are silent:
  * W is stored [V, Dm] (output rows, the usual layout of a linear layer's weight); h and W are
    bf16; the logits are the exact products and sums (float64 here).
  * Ties of the maximum go to the lowest token id (as everywhere else).
  * Node c >= 1 with parent p and token x gets cand_logit[c] = l_p[x]; the root gets NaN.
  * Rows past n_nodes, and every row of a sequence with an error, get max NaN, argmax -1,
    S and A NaN and cand_logit NaN.  Errors: n_nodes outside [0, N] (ERR_NNODES at node 0),
    parents[0] != -1 (ERR_ROOT), parents[i] outside [0, i) (ERR_PARENT), a non-root token
    outside [0, V) (ERR_TOKEN); the smallest (node, code) word wins.
"""

import numpy as np

from .errors import ERR_ROOT, ERR_PARENT, ERR_NNODES, ERR_TOKEN, encode_err


def row_statistics(logits_row):
    """(max, lowest argmax, S = sum exp(l - max), A = sum exp(l - max) (l - max)) in float64."""
    row = np.asarray(logits_row, dtype=np.float64)
    m = row.max()
    am = int(np.flatnonzero(row == m)[0])
    e = np.exp(row - m)
    return m, am, float(e.sum()), float((e * (row - m)).sum())


def lm_head_stats(hidden, W, parents, tokens, n_nodes=None):
    """hidden [B, N, Dm] (bf16 values), W [V, Dm] (bf16 values), parents / tokens int [B, N].

    Returns dict: logits float64 [B, N, V] (for the tests; the GPU never writes them),
    row_max, row_sum, row_ent float64 [B, N], row_argmax int32 [B, N], cand_logit float64
    [B, N], err int32 [B]."""
    hidden = np.asarray(hidden, dtype=np.float64)
    W64 = np.asarray(W, dtype=np.float64)
    B, N, Dm = hidden.shape
    V = W64.shape[0]
    if n_nodes is None:
        n_nodes = np.full(B, N, dtype=np.int64)
    out = {"logits": np.full((B, N, V), np.nan),
           "row_max": np.full((B, N), np.nan), "row_argmax": np.full((B, N), -1, dtype=np.int32),
           "row_sum": np.full((B, N), np.nan), "row_ent": np.full((B, N), np.nan),
           "cand_logit": np.full((B, N), np.nan), "err": np.zeros(B, dtype=np.int32)}
    for b in range(B):
        n = int(n_nodes[b])
        if not 0 <= n <= N:
            out["err"][b] = encode_err(0, ERR_NNODES)
            continue
        problems = []
        if n > 0 and int(parents[b, 0]) != -1:
            problems.append((0, ERR_ROOT))
        for c in range(1, n):
            p = int(parents[b, c])
            if not 0 <= p < c:
                problems.append((c, ERR_PARENT))
            elif not 0 <= int(tokens[b, c]) < V:
                problems.append((c, ERR_TOKEN))
        if problems:
            out["err"][b] = encode_err(*min(problems))
            continue
        if n > 0:
            out["logits"][b, :n] = hidden[b, :n] @ W64.T      # l_i[v] = sum_k W[v, k] h_i[k]
        for i in range(n):
            m, am, S, A = row_statistics(out["logits"][b, i])
            out["row_max"][b, i], out["row_argmax"][b, i] = m, am
            out["row_sum"][b, i], out["row_ent"][b, i] = S, A
        for c in range(1, n):
            out["cand_logit"][b, c] = out["logits"][b, int(parents[b, c]), int(tokens[b, c])]
    return out
