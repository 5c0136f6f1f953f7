"""CPU oracle for the tree-verification step of Medusa/EAGLE-style speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path (the
HIP library and its Python binding) never calls it; the two share no code, helpers or
constants, and this package imports nothing from the HIP side.

Everything is plain NumPy in float64: fp32 and bf16 inputs are upcast exactly, and each
function writes out the plain definition of what the method computes.  The definitions
follow three web pages, cited by title and section:

  [MTP]       "多トークン予測（Medusa・EAGLE）"                          (tech-tldr.com)
  [GLOSSARY]  "Medusa（マルチヘッド投機的デコーディング）"                 (jisaku.com glossary)
  [GUIDE]     "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド"   (qiita.com)

Where the pages leave a step open, each function states the reading it takes.

Pins (tests that tie these functions to something other than themselves) live in
``tests/test_oracle_*.py``; every function here is pinned.
"""

from .errors import (ERR_ROOT, ERR_PARENT, ERR_DEPTH, ERR_NNODES, ERR_PREFIX, ERR_TOKEN,
                     ERR_DRAFTROW, ERR_NONFINITE, ERR_MAP, ERR_RANK, ERR_PROB, encode_err, decode_err)
from .tree import tree_build, pack_mask, unpack_mask
from .attention import tree_attention, tree_attention_row
from .verify import (verify, MODE_GREEDY, MODE_TYPICAL, MODE_REJECT, MODE_WALK,
                     sample_inverse_cdf, residual_after_rejections)
from .heads import medusa_heads
from .assemble import tree_assemble, tree_assemble_rows
from .kv import kv_compact
from .select import tree_select, path_value
from .lm_head import lm_head_stats, row_statistics

__all__ = [
    "ERR_ROOT", "ERR_PARENT", "ERR_DEPTH", "ERR_NNODES", "ERR_PREFIX", "ERR_TOKEN",
    "ERR_DRAFTROW", "ERR_NONFINITE", "ERR_MAP", "ERR_RANK", "ERR_PROB", "encode_err", "decode_err",
    "tree_build", "pack_mask", "unpack_mask", "tree_attention", "tree_attention_row",
    "verify", "MODE_GREEDY", "MODE_TYPICAL", "MODE_REJECT", "MODE_WALK", "sample_inverse_cdf",
    "residual_after_rejections",
    "medusa_heads", "tree_assemble", "tree_assemble_rows", "kv_compact", "tree_select", "path_value", "lm_head_stats", "row_statistics",
]
