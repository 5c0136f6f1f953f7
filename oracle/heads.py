"""Oracle: Medusa heads on the last hidden state, shared LM head, per-head top-k
(test infrastructure only).

What the pages fix:
  * [MTP] section "Medusa：本体に複数の予測ヘッドを足す" and its diagram: several light
    heads sit on the same final hidden state h_t; all of them run in the same single
    forward pass and each predicts a token further ahead.
  * [GUIDE] section "アーキテクチャ：複数ヘッドによる並列トークン予測": each Medusa head is
    a one-layer feed-forward block with a residual connection.
  * [GLOSSARY] section "Medusaの基本アーキテクチャ" (component table and flow): the heads'
    outputs are vocabulary distributions, and the top candidates of each head are combined
    into the candidate tree ("ツリー構造の候補構築").
  * [GUIDE] section "ドラフトヘッドの構成と学習手順": hidden size 4096 and SiLU activation
    for the Llama-3.1-8B-class shapes.

Readings taken where the pages differ or are silent:
  * Head k is a SiLU residual block  z_k = h + SiLU(W_k h)  with no bias, W_k stored as
    [out, in]; the glossary's ReLU / two-layer variant is not used.
  * Every head then goes through one shared LM head: logits_k = W_lm z_k, D_k =
    softmax(logits_k).  A per-head projection would only be a different matrix per head.
  * z_k is kept at full precision (no rounding back to bf16) so that the top-k ranking is
    decided on the exact product.
  * top-k: the k largest logits, in descending order, lower token id first on ties.
"""

import numpy as np


def medusa_heads(h, W_res, W_lm, k):
    """h [B, Dm]; W_res [H, Dm, Dm] ([out, in]); W_lm [V, Dm]; k >= 1.

    Returns a dict: z [B, H, Dm], logits [B, H, V], probs [B, H, V], topk_idx int32
    [B, H, k], topk_prob [B, H, k] and topk_margin [B, H] (the smallest logit gap among the
    k+1 best, i.e. how close the ranking came to changing)."""
    h = np.asarray(h, dtype=np.float64)
    B, Dm = h.shape
    H = W_res.shape[0]
    V = W_lm.shape[0]
    W_lm64 = np.asarray(W_lm, dtype=np.float64)
    z = np.zeros((B, H, Dm))
    for j in range(H):
        a = h @ np.asarray(W_res[j], dtype=np.float64).T       # W_j h for every batch row
        silu = a / (1.0 + np.exp(-a))
        z[:, j, :] = h + silu
    logits = z @ W_lm64.T                                      # [B, H, V]
    probs = np.zeros_like(logits)
    topk_idx = np.zeros((B, H, k), dtype=np.int32)
    topk_prob = np.zeros((B, H, k))
    topk_margin = np.zeros((B, H))
    for b in range(B):
        for j in range(H):
            row = logits[b, j]
            e = np.exp(row - row.max())
            probs[b, j] = e / e.sum()
            order = sorted(range(V), key=lambda v: (-row[v], v))
            best = order[:k]
            topk_idx[b, j] = best
            topk_prob[b, j] = probs[b, j, best]
            ranked = row[order[:k + 1]]
            topk_margin[b, j] = float(np.min(ranked[:-1] - ranked[1:])) if len(ranked) > 1 else np.inf
    return {"z": z, "logits": logits, "probs": probs, "topk_idx": topk_idx,
            "topk_prob": topk_prob, "topk_margin": topk_margin}
