/*
 * spectree.h - C ABI of the tree-verification step of Medusa/EAGLE-style speculative decoding,
 * implemented as hand-written HIP kernels for AMD MI355X (gfx950).
 *
 * The method is described on three web pages, cited below by title and section:
 *   [MTP]       "多トークン予測（Medusa・EAGLE）" (tech-tldr.com)
 *   [GLOSSARY]  "Medusa（マルチヘッド投機的デコーディング）" (jisaku.com glossary)
 *   [GUIDE]     "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド" (qiita.com)
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer unless stated otherwise, allocated and owned by
 *     the caller, row-major with the shape given in brackets.  The library allocates no device
 *     memory on a call path; scratch space comes in through `workspace`.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call validates its scalar
 *     arguments on the host, enqueues its kernels on `stream` and returns without waiting.
 *     Outputs are valid once the stream reaches the call.
 *   - Host-checkable problems (a NULL required pointer, a size out of range, an unsupported
 *     combination, a workspace that is too small) return a non-zero spec_status and enqueue
 *     nothing.  A failed launch returns SPEC_EHIP.
 *   - Problems in the DATA are found on the device and reported per sequence in an `err`
 *     array of error words: 0 = fine, otherwise (node << 8) | code with the codes below.  When
 *     a sequence has several problems the smallest word is reported (lowest node index, then
 *     lowest code); sequence-level problems (node count, prefix length) take node 0 and are
 *     checked first.  A sequence with an error gets the documented neutral outputs.
 *   - Workspaces: query the size with the matching *_workspace() function (0 for a shape the
 *     call does not support: the query applies the call's size checks).  A workspace needs
 *     no initialisation: every call writes each workspace byte it later reads (the only
 *     cross-workgroup counters, those of spec_verify's WALK mode, are zeroed by an earlier
 *     kernel of the same call), so one workspace can be reused by back-to-back calls on one
 *     stream.  Calls that run concurrently need distinct workspaces.
 *   - Codes of the spec_dtype and spec_mode enumerations are passed as plain int arguments
 *     (`dtype`, `mode`), so that any value a caller passes is checked, never assumed valid.
 *   - Limits: N (tree nodes per sequence, padding included) <= 256.
 */
#ifndef SPECTREE_H
#define SPECTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = 1,        /* bad argument: NULL required pointer, size out of range     */
  SPEC_EUNSUPPORTED = 2,  /* well-formed but unsupported: head_dim, dtype, group size   */
  SPEC_EWORKSPACE = 3,    /* workspace NULL or smaller than the *_workspace() size      */
  SPEC_EHIP = 4,          /* a HIP runtime call or a kernel launch failed               */
  SPEC_ESCRATCH = 5       /* the call needs more scratch than spec_verify_static's array */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

typedef enum {
  SPEC_VERIFY_GREEDY = 0,   /* temperature 0: accept iff the token is the argmax          */
  SPEC_VERIFY_TYPICAL = 1,  /* accept iff T[x] >= min(eps, delta * exp(-entropy(T)))     */
  SPEC_VERIFY_REJECT = 2,   /* accept with probability min(1, T[x] / D[x])               */
  SPEC_VERIFY_WALK = 3      /* REJECT made lossless on trees: siblings tried in order      */
} spec_mode;

/* Per-sequence data error codes (low byte of an error word). */
enum {
  SPEC_ERR_ROOT = 1,       /* node 0 must have parent -1                                  */
  SPEC_ERR_PARENT = 2,     /* node i >= 1 must have a parent in [0, i)                    */
  SPEC_ERR_DEPTH = 3,      /* given depth disagrees with the tree, or exceeds max_depth   */
  SPEC_ERR_NNODES = 4,     /* n_nodes[b] outside [0, N]                                   */
  SPEC_ERR_PREFIX = 5,     /* prefix_len[b] < 0, or prefix_len[b] + n_nodes[b] > S_max     */
  SPEC_ERR_TOKEN = 6,      /* candidate token outside [0, V)                              */
  SPEC_ERR_DRAFTROW = 7,   /* draft_row outside [0, R)                                    */
  SPEC_ERR_NONFINITE = 8,  /* a target-logits row that is read holds a NaN or an infinity */
  SPEC_ERR_MAP = 9,        /* t2d entry outside [-1, Vd)                                  */
  SPEC_ERR_RANK = 10,      /* assembly: node deeper than the heads, or sibling rank >= k  */
  SPEC_ERR_PROB = 11       /* selection: a candidate's draft probability is not in [0, 1] */
};

#define SPEC_MAX_NODES 256
#define SPEC_MAX_CANDIDATES 4096

/* Human-readable name of a status code (static storage, never NULL). */
const char* spec_strerror(int status);

/* --------------------------------------------------------------------------------------
 * spec_tree_build - ancestor mask, depths and positions of a batch of candidate trees.
 *
 * [MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる" and [GUIDE] section
 * "Tree Attention：候補を木構造で探索する": each tree node may attend only to its ancestors,
 * which lets every candidate path share one forward pass.  [GLOSSARY] section
 * "デプロイと運用上の考慮事項": batched requests carry their own trees, hence padding + masks.
 *
 *   parents    int32 [B, N]  parent of node i; node 0 is the root (parent -1); a valid tree
 *                            is numbered topologically: parents[i] in [0, i) for i >= 1
 *   depths_in  int32 [B, N]  optional (NULL): depths to validate (SPEC_ERR_DEPTH on mismatch)
 *   prefix_len int32 [B]     optional (NULL = 0): committed prefix length P_b
 *   n_nodes    int32 [B]     optional (NULL = N): valid nodes; rows >= n_nodes are padding
 * Outputs:
 *   mask       uint64 [B, N, W], W = ceil(N / 64): bit (j % 64) of word j / 64 of row i is set
 *                            iff node j is an ancestor of node i or j == i
 *   positions  int32 [B, N]  P_b + depth(i): the rotary position of node i (its KV cache slot
 *                            is P_b + i)
 *   depths     int32 [B, N]  number of proper ancestors
 *   err        int32 [B]     error word
 * Padding rows, and all rows of a sequence with an error, get mask 0, depth -1, position -1.
 * Errors: SPEC_EINVAL if B < 1, N < 1, N > 256 or a required pointer is NULL.
 * ------------------------------------------------------------------------------------ */
spec_status spec_tree_build(const int32_t* parents, const int32_t* depths_in,
                            const int32_t* prefix_len, const int32_t* n_nodes, int B, int N,
                            uint64_t* mask, int32_t* positions, int32_t* depths, int32_t* err,
                            void* stream);

/* --------------------------------------------------------------------------------------
 * spec_tree_assemble - candidate tokens of a predefined tree topology from per-head top-k.
 *
 * [GLOSSARY] section "ツリー構造の候補構築": the candidate tree combines the top candidates
 * of each head on a predefined topology ("Medusa Tree"); e.g. top-3 x top-3 x top-2 gives
 * 18 paths.  The r-th child (counted from 0 in node order) of a node at depth t takes the
 * rank-r candidate of head t:  tokens[b, i] = topk_idx[b, depth(i) - 1, rank(i)].
 *
 *   topk_idx    int32 [B, H, k]  per-head candidates, best first (spec_medusa_heads output)
 *   parents     int32 [N]        topology shared by the batch (same rules as above)
 *   root_tokens int32 [B]        optional (NULL): token of the root (else -1)
 * Outputs:
 *   tokens      int32 [B, N]     candidate token of each node
 *   draft_row   int32 [B, N]     depth(i) - 1: the head (draft row) that proposed node i;
 *                                -1 for the root
 *   err         int32 [B]        error word (the same for every b: the topology is shared);
 *                                on error tokens and draft_row are -1
 * Errors: SPEC_EINVAL if B, N, H, k < 1, N > 256 or a required pointer is NULL.
 * ------------------------------------------------------------------------------------ */
spec_status spec_tree_assemble(const int32_t* topk_idx, const int32_t* parents,
                               const int32_t* root_tokens, int B, int N, int H, int k,
                               int32_t* tokens, int32_t* draft_row, int32_t* err, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_tree_assemble_rows - candidate tokens of a draft tree from per-node draft distributions
 * (EAGLE style): each node's children take the top candidates of the distribution computed at
 * that node.
 *
 * [MTP] section "EAGLE：token ではなく「特徴量」を先読みする": each drafted step gives a
 * candidate distribution through the LM head, and the steps are repeated into a draft tree;
 * [GUIDE] section "Tree Attention：候補を木構造で探索する": several candidates are proposed for
 * one position.  The children of node p, in node order c_0 < c_1 < ..., share the draft row
 * r = draft_row[b, c_0]; child c_j takes the j-th entry of row r ranked by probability, highest
 * first, ties to the lower draft id (-0.0 equals 0.0): tokens[b, c_j] = d2t[id],
 * cand_prob[b, c_j] = draft_probs[b, r, id].
 *
 *   draft_probs float [B, R, Vd]  draft distributions (e.g. one per expanded node)
 *   parents     int32 [B, N]      the tree (rules as in spec_tree_build)
 *   draft_row   int32 [B, N]      row of draft_probs holding node c's distribution's source
 *                                 (the row computed at c's parent; root entry ignored)
 *   d2t         int32 [Vd]        optional (NULL: identity, requires V == Vd): draft id ->
 *                                 target id
 *   n_nodes     int32 [B]         optional (NULL = N); root_tokens int32 [B] optional (NULL: -1)
 *   V                             target vocabulary: every mapped token must lie in [0, V)
 * Outputs:
 *   tokens     int32 [B, N]  candidate token of each node (root: root_tokens[b] or -1)
 *   cand_prob  float [B, N]  draft probability of each node's token (root: 1); it feeds
 *                            spec_tree_select as cand_prob
 *   err        int32 [B]     error word: SPEC_ERR_NNODES, SPEC_ERR_ROOT, SPEC_ERR_PARENT,
 *                            SPEC_ERR_DRAFTROW (row outside [0, R), or a sibling's row differs
 *                            from the first sibling's), SPEC_ERR_RANK (a child ranked past Vd),
 *                            SPEC_ERR_NONFINITE (a NaN in a ranked row, at the first child),
 *                            SPEC_ERR_MAP (d2t gives a token outside [0, V))
 * A sequence with an error, and padding nodes, get token -1 and cand_prob NaN.
 * Workspace: spec_tree_assemble_rows_workspace(B, N, Vd) bytes (per chunk of 8192 draft ids,
 * the chunk's ranked candidates of every node and a NaN flag).
 * Supported: N <= 256, Vd <= 262144.
 * Errors: SPEC_EINVAL (sizes, NULL required pointers, d2t NULL with V != Vd), SPEC_EUNSUPPORTED
 * (Vd), SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t spec_tree_assemble_rows_workspace(int B, int N, int Vd);
spec_status spec_tree_assemble_rows(const float* draft_probs, const int32_t* parents,
                                    const int32_t* draft_row, const int32_t* d2t,
                                    const int32_t* n_nodes, const int32_t* root_tokens, int B,
                                    int N, int R, int Vd, int V, int32_t* tokens,
                                    float* cand_prob, int32_t* err, void* workspace,
                                    size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_tree_attn - tree attention: every node's query attends to the shared committed prefix
 * and to its own ancestors (and itself) under the ancestor mask.
 *
 * [MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる"; [GUIDE] sections
 * "並列検証：ターゲットモデルの1回のforward passで一括確認する" (the KV cache lets all
 * positions be scored in one pass) and "Tree Attention：候補を木構造で探索する".
 *
 *   q          [B, N, Hq, head_dim]        dtype; rotary embedding already applied
 *   k_cache    [B, Hkv, S_max, head_dim]   dtype; slots [0, P_b) hold the prefix, slot P_b + j
 *   v_cache    [B, Hkv, S_max, head_dim]   holds tree node j (written by the caller)
 *   prefix_len int32 [B]                   P_b
 *   tree_mask  uint64 [B, N, ceil(N/64)]   spec_tree_build's mask
 *   n_nodes    int32 [B]                   optional (NULL = N)
 *   scale      softmax scale, positive and finite (1/sqrt(head_dim) for standard attention)
 *   dtype      SPEC_F32 (exact fp32 path) or SPEC_BF16 (MFMA path, fp32 accumulation)
 * Outputs:
 *   out        [B, N, Hq, head_dim] dtype: softmax(scale q.k) v over the visible slots;
 *              query head h reads key/value head h / (Hq / Hkv)
 *   lse        float [B, N, Hq]     optional (NULL): natural-log sum of exp(scale q.k) over the
 *              visible slots (-inf for a row that sees nothing)
 *   err        int32 [B]            optional (NULL): SPEC_ERR_NNODES / SPEC_ERR_PREFIX
 * Rows of padding nodes, rows that see no slot and all rows of a sequence with an error are 0.
 * Supported: head_dim 64 or 128; Hq % Hkv == 0; N <= 256; S_max * head_dim * 2 < 2^31 (the
 * K and V cache of one sequence and KV head below 2 GiB each).
 * Errors: SPEC_EINVAL (sizes, NULL pointers, scale not positive and finite),
 * SPEC_EUNSUPPORTED (head_dim, dtype), SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t spec_tree_attn_workspace(int B, int N, int Hq, int Hkv, int head_dim, int S_max,
                                int dtype);
spec_status spec_tree_attn(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* prefix_len, const uint64_t* tree_mask,
                           const int32_t* n_nodes, int B, int N, int Hq, int Hkv, int head_dim,
                           int S_max, float scale, int dtype, void* out, float* lse,
                           int32_t* err, void* workspace, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_verify - per-node acceptance, longest accepted root-to-node path and bonus token.
 *
 * [GUIDE] section "棄却サンプリング：出力品質を保証する": accept a drafted token x with
 * probability min(1, T[x]/D[x]); on a rejection draw from norm(relu(T - D)); candidates after
 * a rejection are dropped.  [GLOSSARY] section "Medusa-1とMedusa-2の違い": typical
 * acceptance keeps x when T[x] reaches an entropy-based threshold.  [MTP] section
 * "ツリー検証：候補を「木」に束ねて1回で確かめる": the path that passes the longest is kept.
 *
 * Row p of target_logits is the target model's logits at node p; T_p = softmax(row p) is the
 * distribution of p's children.  Node c (parent p, token x = tokens[b, c]) is tested on T_p:
 *   GREEDY   accept iff x == argmax T_p (lowest id on ties)
 *   TYPICAL  accept iff T_p[x] >= min(eps, delta * exp(-H_p)), H_p the entropy of T_p in nats
 *            (delta = +inf gives the fixed threshold eps)
 *   REJECT   accept iff uniforms[b, c] * D[x] < T_p[x], D = draft_probs[b, draft_row[b, c]]
 *            seen on the target vocabulary through t2d
 * A node survives iff it and all its ancestors below the root were accepted.  m = the deepest
 * survivor (lowest index on ties); accept_len = depth(m); path = root .. m.
 *   WALK     the same section's residual rule applied per rejected sibling, which keeps the
 *            output law equal to the target's on branching trees (REJECT keeps it on chains
 *            only).  From p = root: the children of p, in index order, are tested against a
 *            running R (first T_p): accept iff uniforms[b, c] * D[x] < R[x]; a rejection sets
 *            R = norm(relu(R - D)) (zero mass: every later sibling is rejected).  The first
 *            accepted child becomes p; the walk ends at m when all children of m (or none)
 *            are rejected.  All children of a node must share one draft row (else
 *            SPEC_ERR_DRAFTROW at the first child that differs).  node_accept marks the path.
 * Bonus token, drawn
 * with uniforms[b, 0] by inverse CDF (smallest t whose running sum from token 0 exceeds u * Z):
 *   GREEDY   argmax T_m
 *   TYPICAL  a draw from T_m
 *   REJECT   if m has children: a draw from norm(relu(T_m - D)), D the draft row of m's
 *            lowest-index child (T_m if that residual is all zero); else a draw from T_m.
 *   WALK     the running R of m after all its children were rejected (T_m if it has summed
 *            to zero, or if m has no child).
 *
 *   target_logits float [B, N, V]
 *   draft_probs   float [B, R, Vd]  draft distributions (REJECT, WALK; else may be NULL)
 *   draft_row     int32 [B, N]      row of draft_probs that proposed node c (REJECT, WALK)
 *   t2d           int32 [V]         optional (NULL: identity, requires Vd == V): target id ->
 *                                   draft id, -1 where the draft vocabulary lacks the token
 *   tokens        int32 [B, N]      candidate token of each node (node 0's is ignored)
 *   parents       int32 [B, N]      tree (rules as in spec_tree_build)
 *   n_nodes       int32 [B]         optional (NULL = N)
 *   uniforms      float [B, N]      U[0, 1) draws: column 0 for the bonus, column c for node c
 *   max_depth     length of path minus one; a valid node deeper than this is SPEC_ERR_DEPTH
 * Outputs:
 *   accept_len  int32 [B]; path int32 [B, max_depth + 1] (-1 padded); bonus_token int32 [B];
 *   node_accept uint8 [B, N] optional (NULL): per-node test result (root 1, padding 0;
 *               WALK: 1 on the path);
 *   err         int32 [B].
 * A sequence with n_nodes 0, or with an error, gets accept_len 0, path all -1, bonus -1 and
 * node_accept all 0.
 * Supported: V <= 1048576 (256 chunks of 4096 logits in the bonus draw).
 * Errors: SPEC_EINVAL (sizes, NULL pointers, REJECT without draft arrays, t2d NULL with
 * Vd != V, TYPICAL with a NaN eps or delta), SPEC_EUNSUPPORTED (V), SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t spec_verify_workspace(int B, int N, int V);
spec_status spec_verify(const float* target_logits, const float* draft_probs,
                        const int32_t* draft_row, const int32_t* t2d, const int32_t* tokens,
                        const int32_t* parents, const int32_t* n_nodes, const float* uniforms,
                        int B, int N, int V, int R, int Vd, int max_depth, int mode,
                        float eps, float delta, int32_t* accept_len, int32_t* path,
                        int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                        void* workspace, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_verify_static - spec_verify without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc).
 *
 * Arguments, outputs, rules and data errors are exactly spec_verify's (same kernels).  The
 * scratch lives in a fixed device array of the library, SPEC_VERIFY_STATIC_MAX_BYTES per GPU,
 * which each GPU the library runs on holds until the process ends; this call allocates and
 * frees nothing.  spec_verify_static_bytes() gives the scratch a call of that size needs (it
 * is at most spec_verify_workspace()).  Every call on one GPU uses that GPU's array and leaves
 * its own contents there: calls that overlap on one GPU (on different streams, or from
 * different host threads) race and give undefined results.  No call relies on the array's
 * previous contents (every byte read is written earlier in the same call).  `stream` must
 * belong to the current device (NULL: the current device's null stream).
 * Errors: as spec_verify, plus SPEC_ESCRATCH when spec_verify_static_bytes() exceeds
 * SPEC_VERIFY_STATIC_MAX_BYTES (e.g. batch 8 at a vocabulary near 10^6), SPEC_EINVAL when
 * `stream` belongs to another device, SPEC_EHIP when the array's address cannot be found.
 * ------------------------------------------------------------------------------------ */
#define SPEC_VERIFY_STATIC_MAX_BYTES ((size_t)16 << 20)
size_t spec_verify_static_bytes(int B, int N, int V);
spec_status spec_verify_static(const float* target_logits, const float* draft_probs,
                               const int32_t* draft_row, const int32_t* t2d, const int32_t* tokens,
                               const int32_t* parents, const int32_t* n_nodes, const float* uniforms,
                               int B, int N, int V, int R, int Vd, int max_depth, int mode,
                               float eps, float delta, int32_t* accept_len, int32_t* path,
                               int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                               void* stream);

/* --------------------------------------------------------------------------------------
 * spec_tree_select - dynamic tree: keep the best N-node subtree of a drafted candidate tree.
 *
 * [MTP] section "ツリー検証：候補を「木」に束ねて1回で確かめる": a larger tree raises the
 * expected accepted length but costs verification work; EAGLE-2's dynamic tree shapes the tree
 * by the context's confidence.  [GLOSSARY] section "EAGLE: Medusaの発展形" and [GUIDE] section
 * "EAGLE-1/2からの進化" name the same context-aware tree.  The rule taken: a candidate's value
 * is the product of the draft probabilities on its path from the root (the root counts 1;
 * float64 products of the float32 inputs, multiplied root first); the root and the N - 1 other
 * candidates of largest value are kept, ties to the lower candidate index.  With every
 * probability in [0, 1] the kept set contains each member's parent.  Kept candidates are
 * written in candidate order (so the output is numbered topologically) with renumbered parents.
 *
 *   cand_parents int32 [B, C]  candidate tree: candidate 0 the root (parent -1), parents[i] in
 *                              [0, i) for i >= 1
 *   cand_prob    float [B, C]  draft probability of each candidate's token (root entry unused)
 *   n_cand       int32 [B]     optional (NULL = C): valid candidates per sequence
 *   cand_tokens  int32 [B, C]  optional (NULL): carried to `tokens`
 *   cand_row     int32 [B, C]  optional (NULL): carried to `draft_row` unchanged (the draft rows
 *                              stay those of the candidate pool)
 * Outputs (every entry written; entries j >= n_nodes[b] are -1):
 *   sel          int32 [B, N]  candidate index of output node j
 *   parents      int32 [B, N]  parent of output node j among the output nodes (-1: root)
 *   tokens       int32 [B, N]  given iff cand_tokens is given
 *   draft_row    int32 [B, N]  given iff cand_row is given
 *   n_nodes      int32 [B]     min(n_cand[b], N), 0 on error
 *   err          int32 [B]     error word: SPEC_ERR_NNODES (n_cand outside [0, C], at node 0),
 *                              SPEC_ERR_ROOT, SPEC_ERR_PARENT, SPEC_ERR_PROB (a non-root
 *                              probability that is NaN or outside [0, 1]); a sequence with an
 *                              error keeps nothing
 * The outputs feed spec_tree_build (parents, n_nodes) and spec_verify (tokens, draft_row).
 * All pointers are device memory; no workspace.
 * Supported: 1 <= C <= 4096, 1 <= N <= 256.
 * Errors: SPEC_EINVAL (sizes, NULL required pointer, exactly one of cand_tokens / tokens or of
 * cand_row / draft_row NULL).
 * ------------------------------------------------------------------------------------ */
spec_status spec_tree_select(const int32_t* cand_parents, const float* cand_prob,
                             const int32_t* n_cand, const int32_t* cand_tokens,
                             const int32_t* cand_row, int B, int C, int N, int32_t* sel,
                             int32_t* parents, int32_t* tokens, int32_t* draft_row,
                             int32_t* n_nodes, int32_t* err, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_lm_head_stats - the target's LM head fused with the row statistics verification reads.
 *
 * [GUIDE] section "並列検証：ターゲットモデルの1回のforward passで一括確認する": one target pass
 * gives every tree node's distribution T_p = softmax(W h_p); [GUIDE] section
 * "ドラフトヘッドの構成と学習手順" gives the shapes (hidden 4096, vocabulary 128256).  Only a few
 * numbers of each row are read by verification, so the logits are reduced as they are produced
 * and never written:
 *   l_p[v]      = sum_k W[v, k] h_p[k]      (bf16 inputs, fp32 accumulation)
 *   row_max     = max_v l_p[v],  row_argmax = the lowest v holding it
 *   row_sum     = sum_v exp(l_p[v] - row_max)                     (T_p[x] = exp(l_p[x] - max) / S)
 *   row_ent     = sum_v exp(l_p[v] - row_max) (l_p[v] - row_max)  (entropy = ln S - row_ent / S)
 *   cand_logit  = l_parent(c)[tokens[c]] for every non-root node c (NaN for the root)
 *
 *   hidden   bf16 [B, N, Dm]  the target's last hidden state at each tree node (16-byte aligned)
 *   W        bf16 [V, Dm]     the target's LM head ([out, in]; 16-byte aligned)
 *   parents  int32 [B, N], tokens int32 [B, N] (node c's candidate token), n_nodes int32 [B]
 *            (optional, NULL = N): the same tree rules as spec_tree_build
 * Outputs: row_max float [B, N], row_argmax int32 [B, N], row_sum, row_ent double [B, N],
 *   cand_logit float [B, N], err int32 [B]: SPEC_ERR_NNODES, SPEC_ERR_ROOT, SPEC_ERR_PARENT,
 *   SPEC_ERR_TOKEN (a non-root token outside [0, V)).  Rows past n_nodes and every row of a
 *   sequence with an error get NaN (argmax -1).
 * The workspace (spec_lm_head_stats_workspace bytes) holds one partial per (row, 64 tokens) and
 * a copy of the hidden states in the order the matrix-core fragments read them.
 * Supported: N <= 256, B * N <= 4096, Dm a multiple of 128.
 * Errors: SPEC_EINVAL (sizes, NULL pointers), SPEC_EUNSUPPORTED (N, B * N, Dm, alignment),
 * SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t spec_lm_head_stats_workspace(int B, int N, int Dm, int V);
spec_status spec_lm_head_stats(const void* hidden, const void* W, const int32_t* parents,
                               const int32_t* tokens, const int32_t* n_nodes, int B, int N, int Dm,
                               int V, float* row_max, int32_t* row_argmax, double* row_sum,
                               double* row_ent, float* cand_logit, int32_t* err, void* workspace,
                               size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_verify_greedy_stats - greedy verification from spec_lm_head_stats' statistics, so that a
 * temperature-0 round never materialises the N x V logits.
 *
 * The GREEDY rule of spec_verify on the row arg-maxima alone ([GUIDE] section "結論・成果"
 * quotes speed-ups at temperature 0, where T_p collapses to its lowest-id argmax): node c
 * (parent p, token x) is accepted iff x == row_argmax[b, p]; a node survives iff every node on
 * its path below the root was accepted; m = the deepest survivor (lowest index on ties);
 * accept_len = depth(m), path = root .. m, bonus_token = row_argmax[b, m].
 *
 *   row_argmax  int32 [B, N]  spec_lm_head_stats' output; tokens, parents int32 [B, N];
 *   n_nodes     int32 [B] optional (NULL = N); max_depth and V as for spec_verify
 * Outputs: accept_len [B], path [B, max_depth + 1], bonus_token [B], node_accept uint8 [B, N]
 *   (optional, NULL), err [B] - exactly as spec_verify in GREEDY mode (errors SPEC_ERR_NNODES,
 *   ROOT, PARENT, DEPTH, TOKEN; a sequence with n_nodes 0 or an error gets accept_len 0,
 *   path -1, bonus -1, node_accept 0).  No workspace.
 * Supported: N <= 256.
 * Errors: SPEC_EINVAL (sizes, NULL required pointers).
 * ------------------------------------------------------------------------------------ */
spec_status spec_verify_greedy_stats(const int32_t* row_argmax, const int32_t* tokens,
                                     const int32_t* parents, const int32_t* n_nodes, int B, int N,
                                     int V, int max_depth, int32_t* accept_len, int32_t* path,
                                     int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                                     void* stream);

/* --------------------------------------------------------------------------------------
 * spec_verify_lm_head - greedy, typical, rejection-sampling or sibling-residual-walk
 * verification straight from the target's hidden states: spec_lm_head_stats' statistics, then
 * spec_verify's rule on them (GREEDY and TYPICAL without storing the N x V logits).
 *
 * The rules are spec_verify's: GREEDY accepts node c (parent p, token x) iff x is p's lowest
 * argmax; TYPICAL iff T_p[x] = exp(l_p[x] - max_p) / S_p >= min(eps, delta exp(-H_p)) with
 * H_p = ln S_p - A_p / S_p; REJECT iff uniforms[b, c] * D[x] < T_p[x]; survival, the deepest
 * survivor m and the path as spec_verify.  Bonus token, by inverse CDF with u = uniforms[b, 0]
 * (smallest t whose running sum from token 0 exceeds u Z): GREEDY the argmax of row m; TYPICAL,
 * and REJECT when m has no child, a draw from T_m - the 64-token tile holding u Z is found from
 * the per-tile sums of the statistics pass and only that tile's logits are recomputed; REJECT
 * when m has children, a draw from norm(relu(T_m - D)), D the draft row of m's lowest-index
 * child (T_m if that residual is zero) - in REJECT mode the statistics pass also keeps every
 * row's fp32 logits in the workspace, and the draw scans row m's 64-token tile sums, then one
 * tile.  WALK: the statistics pass stores every row's fp32 logits in the workspace and
 * spec_verify(WALK) runs on them (same outputs and errors as spec_verify on those logits).
 * [GUIDE] sections "並列検証：ターゲットモデルの1回のforward passで一括確認する" and
 * "棄却サンプリング：出力品質を保証する"; [GLOSSARY] section "Medusa-1とMedusa-2の違い".
 *
 *   hidden, W, parents, tokens, n_nodes, B, N, Dm, V  as spec_lm_head_stats
 *   uniforms float [B, N]; draft_probs, draft_row, t2d, R, Vd (REJECT, WALK; else may be NULL),
 *   max_depth, eps, delta  as spec_verify
 * Outputs: accept_len [B], path [B, max_depth + 1], bonus_token [B], node_accept uint8 [B, N]
 *   (optional), err [B]: as spec_verify (SPEC_ERR_NNODES, ROOT, PARENT, DEPTH, TOKEN, DRAFTROW,
 *   MAP, and WALK's NONFINITE).  Workspace: spec_verify_lm_head_workspace(B, N, Dm, V, mode)
 *   bytes (REJECT's and WALK's include B * N * V fp32 logits; WALK's also spec_verify's own).
 * Supported: all four modes, N <= 256, B * N <= 4096, Dm a multiple of 128.
 * Errors: SPEC_EINVAL (sizes, NULL pointers, NaN eps or delta, REJECT or WALK without draft
 * arrays, t2d NULL with Vd != V), SPEC_EUNSUPPORTED (mode, sizes, alignment), SPEC_EWORKSPACE;
 * WALK also returns what spec_verify returns for its call (after the statistics pass ran).
 * ------------------------------------------------------------------------------------ */
size_t spec_verify_lm_head_workspace(int B, int N, int Dm, int V, int mode);
spec_status spec_verify_lm_head(const void* hidden, const void* W, const int32_t* tokens,
                                const int32_t* parents, const int32_t* n_nodes, const float* uniforms,
                                const float* draft_probs, const int32_t* draft_row, const int32_t* t2d,
                                int B, int N, int Dm, int V, int R, int Vd, int max_depth,
                                int mode, float eps, float delta, int32_t* accept_len,
                                int32_t* path, int32_t* bonus_token, uint8_t* node_accept,
                                int32_t* err, void* workspace, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_kv_compact - KV-cache compaction that closes a verification round.
 *
 * [GUIDE] section "Speculative Decodingの動作原理を理解する": decoding repeats draft, one
 * verifying pass of the target model over the KV cache, and rejection sampling; every
 * candidate after a rejected one is discarded.  With tree node i's K/V at cache slot P + i
 * (P = prefix_len[b], node 0 the root), the root and the accepted path are committed: for
 * j = 1..accept_len[b], node path[b, j] moves from slot P + path[b, j] to slot P + j, in every
 * layer, KV head and both caches, and the new prefix length is P + accept_len[b] + 1.  Other
 * slots keep their contents.  A sequence with err[b] != 0, or whose path is not a root-first
 * chain of increasing node indices ending inside the cache (path[b, 0] == 0,
 * path[b, j] > path[b, j - 1], P + path[b, accept_len] < S_max, 0 <= accept_len <= max_depth),
 * is left unchanged (its new prefix length is P); this is not reported as an error.
 *
 *   k_cache, v_cache  L layers of [B, Hkv, S_max, head_dim] elements of `dtype`, layer l at
 *                     element offset l * layer_stride (ignored when L == 1); updated in place
 *   prefix_len        int32 [B]
 *   prefix_len_out    int32 [B] new prefix lengths, or NULL; must not alias prefix_len
 *   path, accept_len  as written by spec_verify (path rows of max_depth + 1 entries)
 *   err               int32 [B] as written by spec_verify, or NULL (no errors)
 * All pointers are device memory.  No workspace.
 * Supported: dtype BF16 or F32 with head_dim * element size a multiple of 16 bytes and at most
 * 1024; 16-byte aligned caches and layer stride.
 * Errors: SPEC_EINVAL (NULL pointers, sizes, layer_stride below one layer when L > 1,
 * prefix_len_out == prefix_len), SPEC_EUNSUPPORTED (dtype, head_dim, alignment).
 * ------------------------------------------------------------------------------------ */
spec_status spec_kv_compact(void* k_cache, void* v_cache, size_t layer_stride, int L,
                            const int32_t* prefix_len, int32_t* prefix_len_out,
                            const int32_t* path, const int32_t* accept_len, const int32_t* err,
                            int B, int Hkv, int S_max, int head_dim, int max_depth,
                            int dtype, void* stream);

/* --------------------------------------------------------------------------------------
 * spec_medusa_heads - Medusa heads on the last hidden state, shared LM head, per-head top-k.
 *
 * [MTP] section "Medusa：本体に複数の予測ヘッドを足す" (several light heads on the same h_t,
 * all in one forward pass); [GUIDE] section "アーキテクチャ：複数ヘッドによる並列トークン予測"
 * (each head: one feed-forward layer with a residual connection); [GLOSSARY] section
 * "Medusaの基本アーキテクチャ" (heads emit vocabulary distributions whose top candidates
 * build the tree).
 *
 *   z_j       = h + SiLU(W_res[j] h)      (no bias; W_res[j] stored [out, in]); kept in fp32
 *   logits_j  = W_lm z_j                  (the shared LM head, fp32 accumulation)
 *   D_j       = softmax(logits_j)
 *
 *   h        bf16 [B, Dm];  W_res bf16 [H, Dm, Dm];  W_lm bf16 [V, Dm]
 * Outputs:
 *   topk_idx    int32 [B, H, k]  the k largest logits of head j, descending, lower id on ties
 *   topk_prob   float [B, H, k]  D_j at those ids
 *   draft_probs float [B, H, V]  optional (NULL): D_j
 * Supported: B <= 16, B * H <= 64, Dm % 128 == 0, 1 <= k <= 64, k <= V.
 * Errors: SPEC_EINVAL, SPEC_EUNSUPPORTED, SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------------------ */
size_t spec_medusa_heads_workspace(int B, int H, int Dm, int V, int k);
spec_status spec_medusa_heads(const void* h, const void* W_res, const void* W_lm, int B, int H,
                              int Dm, int V, int k, int32_t* topk_idx, float* topk_prob,
                              float* draft_probs, void* workspace, size_t ws_bytes,
                              void* stream);


#ifdef __cplusplus
}
#endif

#endif /* SPECTREE_H */
