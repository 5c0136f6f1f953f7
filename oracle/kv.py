"""Oracle: KV-cache compaction that closes a verification round (test infrastructure only).

[GUIDE] section "Speculative Decodingの動作原理を理解する": decoding repeats a cycle of drafting,
one verifying forward pass of the target model and rejection sampling; the verifying pass gets
the distributions at every candidate position at once because of the KV cache (subsection
"並列検証：ターゲットモデルの1回のforward passで一括確認する"), and every candidate after a
rejected one is discarded (subsection "棄却サンプリング：出力品質を保証する", the note).  So
after verification only the committed tokens may keep their K/V in the cache, contiguous after
the prefix, before the next cycle's pass appends the next tree.

Reading (the pages do not spell out this bookkeeping): tree node i's K/V sits at cache slot
P + i (P = prefix length), node 0 being the root, the token committed by the previous round.
The root and the accepted path path[1..a] (a = accept_len) are committed: node path[j] moves
from slot P + path[j] to slot P + j for j = 1..a, and the prefix length becomes P + a + 1.
Every other slot keeps what it held (the next round overwrites the slots past the prefix).  A
sequence whose verification reported an error, or whose path is not a root-first chain of
increasing node indices inside the cache, is left as it was.
"""

import numpy as np


def path_is_valid(path_b, a, P, S_max):
    """The checks applied before a sequence is compacted (see the module's reading)."""
    if a < 0 or a + 1 > len(path_b) or P < 0:
        return False
    chain = [int(x) for x in path_b[:a + 1]]
    if chain[0] != 0:
        return False
    for j in range(1, a + 1):
        if chain[j] <= chain[j - 1]:
            return False
    return P + chain[a] < S_max


def kv_compact(k_cache, v_cache, prefix_len, path, accept_len, err=None):
    """Compact the accepted path's K/V after the prefix, for every layer.

    k_cache, v_cache : [L, B, Hkv, S_max, d] arrays (any dtype; slots are copied exactly)
    prefix_len       : [B] int prefix lengths P_b before the round
    path             : [B, max_depth + 1] node indices root..m, -1 padded
    accept_len       : [B] accepted path length a_b (depth of m)
    err              : [B] verification error words, or None (no errors)

    Returns (k_new, v_new, prefix_len_new); the inputs are not modified.
    """
    k_new = np.array(k_cache, copy=True)
    v_new = np.array(v_cache, copy=True)
    P_new = np.array(prefix_len, dtype=np.int64, copy=True)
    B = k_new.shape[1]
    S_max = k_new.shape[3]
    for b in range(B):
        if err is not None and int(err[b]) != 0:
            continue
        a = int(accept_len[b])
        P = int(prefix_len[b])
        if not path_is_valid(path[b], a, P, S_max):
            continue
        # every source slot is read (from the unmodified input) before any slot is written: a
        # destination P + j may be the source of an earlier node of the path
        k_rows = [k_cache[:, b, :, P + int(path[b, j]), :].copy() for j in range(1, a + 1)]
        v_rows = [v_cache[:, b, :, P + int(path[b, j]), :].copy() for j in range(1, a + 1)]
        for j in range(1, a + 1):
            k_new[:, b, :, P + j, :] = k_rows[j - 1]
            v_new[:, b, :, P + j, :] = v_rows[j - 1]
        P_new[b] = P + a + 1
    return k_new, v_new, P_new.astype(np.int32)
