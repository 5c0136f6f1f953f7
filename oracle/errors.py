"""Per-sequence error codes of the oracle (test infrastructure only).

An error word is ``(node << 8) | code``; 0 means no problem.  When a sequence has several
problems the reported word is the smallest one: the lowest node index first, then the
lowest code.  Sequence-level problems (node count, prefix length) are attached to node 0
and are checked before any per-node rule.

The pages define no error handling; these codes are this project's own contract, written
here independently of the HIP library's header.
"""

ERR_ROOT = 1        # node 0 must have parent -1
ERR_PARENT = 2      # node i >= 1 must have a parent in [0, i) (topological numbering)
ERR_DEPTH = 3       # a given depth disagrees with the tree, or exceeds the path buffer
ERR_NNODES = 4      # valid-node count outside [0, N]
ERR_PREFIX = 5      # prefix length < 0, or prefix + nodes exceeds the KV cache
ERR_TOKEN = 6       # candidate token outside [0, V)
ERR_DRAFTROW = 7    # draft row index outside [0, R)
ERR_NONFINITE = 8   # a logits row that is read holds a NaN or an infinity
ERR_MAP = 9         # target->draft map entry outside [-1, Vd)
ERR_RANK = 10       # tree assembly: a node's depth or sibling rank exceeds the heads' top-k
ERR_PROB = 11       # tree selection: a candidate's draft probability is not a number in [0, 1]


def encode_err(node, code):
    return (int(node) << 8) | int(code)


def decode_err(word):
    word = int(word)
    return word >> 8, word & 0xFF
