"""ctypes declarations of libspectree's exported functions (the C ABI of include/spectree.h
and the internal entry points of csrc/internal.h).  No torch: the host-sanitised library of
the CPU tests is driven through this module alone."""

import ctypes

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t


def declare(L):
    """Set the argument and result types of every exported function on the CDLL ``L``."""
    L.spec_strerror.restype = ctypes.c_char_p
    L.spec_strerror.argtypes = [_I]
    L.spec_tree_build.restype = _I
    L.spec_tree_build.argtypes = [_P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P]
    L.spec_tree_assemble.restype = _I
    L.spec_tree_assemble.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P]
    L.spec_tree_assemble_rows_workspace.restype = _Z
    L.spec_tree_assemble_rows_workspace.argtypes = [_I, _I, _I]
    L.spec_tree_assemble_rows.restype = _I
    L.spec_tree_assemble_rows.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]
    L.spec_tree_select.restype = _I
    L.spec_tree_select.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
    L.spec_lm_head_stats_workspace.restype = _Z
    L.spec_lm_head_stats_workspace.argtypes = [_I, _I, _I, _I]
    L.spec_lm_head_stats.restype = _I
    L.spec_lm_head_stats.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]
    L.spec_verify_greedy_stats.restype = _I
    L.spec_verify_greedy_stats.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.spec_verify_lm_head_workspace.restype = _Z
    L.spec_verify_lm_head_workspace.argtypes = [_I, _I, _I, _I, _I]
    L.spec_verify_lm_head.restype = _I
    L.spec_verify_lm_head.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                      _F, _F, _P, _P, _P, _P, _P, _P, _Z, _P]
    L.spec_tree_attn_workspace.restype = _Z
    L.spec_tree_attn_workspace.argtypes = [_I, _I, _I, _I, _I, _I, _I]
    L.spec_tree_attn.restype = _I
    L.spec_tree_attn.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                                 _P, _Z, _P]
    L.spec_verify_static_bytes.restype = _Z
    L.spec_verify_static_bytes.argtypes = [_I, _I, _I]
    L.spec_verify_static.restype = _I
    L.spec_verify_static.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F,
                                     _P, _P, _P, _P, _P, _P]
    L.spec_verify_workspace.restype = _Z
    L.spec_verify_workspace.argtypes = [_I, _I, _I]
    L.spec_verify.restype = _I
    L.spec_verify.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F,
                              _P, _P, _P, _P, _P, _P, _Z, _P]
    L.spec_medusa_heads_workspace.restype = _Z
    L.spec_medusa_heads_workspace.argtypes = [_I, _I, _I, _I, _I]
    L.spec_medusa_heads.restype = _I
    L.spec_medusa_heads.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]
    L.spec_kv_compact.restype = _I
    L.spec_kv_compact.argtypes = [_P, _P, _Z, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
    L.spec_prof_enable.restype = None
    L.spec_prof_enable.argtypes = [_I]
    L.spec_prof_reset.restype = None
    L.spec_prof_reset.argtypes = []
    L.spec_prof_read.restype = _I
    L.spec_prof_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int64)]
    L.spec_internal_tune.restype = _I
    L.spec_internal_tune.argtypes = [ctypes.c_char_p, _I]
    return L


def load(path):
    return declare(ctypes.CDLL(path))
