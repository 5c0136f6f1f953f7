"""Thin ctypes binding over libspectree.so (the C ABI in include/spectree.h).

Argument marshalling only: every function here checks tensor shapes, dtypes and devices,
allocates the output tensors, and passes raw device pointers plus torch's current HIP stream
to the library.  All computation happens in the library's HIP kernels.  There is no fallback:
if the library is missing or the device is not a GPU, calls raise.
"""

import ctypes
import os

import torch

from . import abi

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspectree.so")

SPEC_F32, SPEC_BF16 = 0, 1
GREEDY, TYPICAL, REJECT, WALK = 0, 1, 2, 3
MODES = {"greedy": GREEDY, "typical": TYPICAL, "reject": REJECT, "walk": WALK}

_lib = None


class SpecError(RuntimeError):
    pass


def lib():
    """Load libspectree.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SpecError(f"{LIB_PATH} is missing: build it with "
                        "`python -m tree_attention_verification_spec_amd.build`")
    _lib = abi.load(LIB_PATH)
    return _lib


def _check(status, what):
    if status != 0:
        raise SpecError(f"{what}: {lib().spec_strerror(status).decode()} (status {status})")


def _ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise SpecError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise SpecError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SpecError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SpecError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace(nbytes, device, fill=None):
    """A workspace buffer of ``nbytes`` bytes on ``device``.  The library needs no
    initialisation (every call writes each workspace byte it later reads), so by default the
    bytes are whatever the allocator hands out; ``fill`` sets every byte to that value."""
    t = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if fill is not None:
        t.fill_(int(fill))
    return t


# ----------------------------------------------------------------------------- tree

def spec_tree_build(parents, depths_in=None, prefix_len=None, n_nodes=None, out=None, stream=None):
    B, N = parents.shape
    dev = parents.device
    W = (N + 63) // 64
    if out is None:
        out = {"mask": torch.empty((B, N, W), dtype=torch.int64, device=dev),
               "positions": torch.empty((B, N), dtype=torch.int32, device=dev),
               "depths": torch.empty((B, N), dtype=torch.int32, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib().spec_tree_build(
        _ptr(parents, torch.int32, (B, N), "parents"), _ptr(depths_in, torch.int32, (B, N), "depths_in"),
        _ptr(prefix_len, torch.int32, (B,), "prefix_len"), _ptr(n_nodes, torch.int32, (B,), "n_nodes"),
        B, N, _ptr(out["mask"], torch.int64, (B, N, W), "mask"),
        _ptr(out["positions"], torch.int32, (B, N), "positions"),
        _ptr(out["depths"], torch.int32, (B, N), "depths"), _ptr(out["err"], torch.int32, (B,), "err"),
        _stream(stream)), "spec_tree_build")
    return out


def spec_tree_assemble(topk_idx, parents, root_tokens=None, out=None, stream=None):
    B, H, k = topk_idx.shape
    N = parents.shape[0]
    dev = topk_idx.device
    if out is None:
        out = {"tokens": torch.empty((B, N), dtype=torch.int32, device=dev),
               "draft_row": torch.empty((B, N), dtype=torch.int32, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib().spec_tree_assemble(
        _ptr(topk_idx, torch.int32, (B, H, k), "topk_idx"), _ptr(parents, torch.int32, (N,), "parents"),
        _ptr(root_tokens, torch.int32, (B,), "root_tokens"), B, N, H, k,
        _ptr(out["tokens"], torch.int32, (B, N), "tokens"),
        _ptr(out["draft_row"], torch.int32, (B, N), "draft_row"),
        _ptr(out["err"], torch.int32, (B,), "err"), _stream(stream)), "spec_tree_assemble")
    return out


def tree_assemble_rows_workspace_bytes(B, N, Vd):
    return int(lib().spec_tree_assemble_rows_workspace(B, N, Vd))


def spec_tree_assemble_rows(draft_probs, parents, draft_row, d2t=None, V=None, n_nodes=None, root_tokens=None,
                            out=None, ws=None, stream=None):
    """EAGLE-style assembly: each node's children take the top candidates of their draft row."""
    B, R, Vd = draft_probs.shape
    N = parents.shape[1]
    dev = draft_probs.device
    if V is None:
        V = Vd
    if out is None:
        out = {"tokens": torch.empty((B, N), dtype=torch.int32, device=dev),
               "cand_prob": torch.empty((B, N), dtype=torch.float32, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(tree_assemble_rows_workspace_bytes(B, N, Vd), dev)
    _check(lib().spec_tree_assemble_rows(
        _ptr(draft_probs, torch.float32, (B, R, Vd), "draft_probs"), _ptr(parents, torch.int32, (B, N), "parents"),
        _ptr(draft_row, torch.int32, (B, N), "draft_row"), _ptr(d2t, torch.int32, (Vd,), "d2t"),
        _ptr(n_nodes, torch.int32, (B,), "n_nodes"), _ptr(root_tokens, torch.int32, (B,), "root_tokens"),
        B, N, R, Vd, int(V), _ptr(out["tokens"], torch.int32, (B, N), "tokens"),
        _ptr(out["cand_prob"], torch.float32, (B, N), "cand_prob"), _ptr(out["err"], torch.int32, (B,), "err"),
        _ptr(ws, None, None, "workspace"), ws.numel(), _stream(stream)), "spec_tree_assemble_rows")
    return out


def spec_tree_select(cand_parents, cand_prob, N, n_cand=None, cand_tokens=None, cand_row=None, out=None,
                     stream=None):
    B, C = cand_parents.shape
    dev = cand_parents.device
    if out is None:
        out = {"sel": torch.empty((B, N), dtype=torch.int32, device=dev),
               "parents": torch.empty((B, N), dtype=torch.int32, device=dev),
               "tokens": torch.empty((B, N), dtype=torch.int32, device=dev) if cand_tokens is not None else None,
               "draft_row": torch.empty((B, N), dtype=torch.int32, device=dev) if cand_row is not None else None,
               "n_nodes": torch.empty((B,), dtype=torch.int32, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib().spec_tree_select(
        _ptr(cand_parents, torch.int32, (B, C), "cand_parents"), _ptr(cand_prob, torch.float32, (B, C), "cand_prob"),
        _ptr(n_cand, torch.int32, (B,), "n_cand"), _ptr(cand_tokens, torch.int32, (B, C), "cand_tokens"),
        _ptr(cand_row, torch.int32, (B, C), "cand_row"), B, C, int(N),
        _ptr(out["sel"], torch.int32, (B, N), "sel"), _ptr(out["parents"], torch.int32, (B, N), "parents"),
        _ptr(out.get("tokens"), torch.int32, (B, N), "tokens"),
        _ptr(out.get("draft_row"), torch.int32, (B, N), "draft_row"),
        _ptr(out["n_nodes"], torch.int32, (B,), "n_nodes"), _ptr(out["err"], torch.int32, (B,), "err"),
        _stream(stream)), "spec_tree_select")
    return out


# ----------------------------------------------------------------------------- attention

def tree_attn_workspace_bytes(B, N, Hq, Hkv, d, S_max, dtype):
    code = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    return int(lib().spec_tree_attn_workspace(B, N, Hq, Hkv, d, S_max, code))


def spec_tree_attn(q, k_cache, v_cache, prefix_len, tree_mask, n_nodes=None, scale=None, out=None,
                   lse=None, err=None, ws=None, stream=None):
    B, N, Hq, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    dt = q.dtype
    code = {torch.bfloat16: SPEC_BF16, torch.float32: SPEC_F32}.get(dt)
    if code is None:
        raise SpecError("q must be bfloat16 or float32")
    if scale is None:
        scale = d ** -0.5
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    if err is None:
        err = torch.empty((B,), dtype=torch.int32, device=dev)
    need = tree_attn_workspace_bytes(B, N, Hq, Hkv, d, S_max, dt)
    if ws is None:
        ws = workspace(need, dev)
    W = (N + 63) // 64
    _check(lib().spec_tree_attn(
        _ptr(q, dt, None, "q"), _ptr(k_cache, dt, (B, Hkv, S_max, d), "k_cache"),
        _ptr(v_cache, dt, (B, Hkv, S_max, d), "v_cache"), _ptr(prefix_len, torch.int32, (B,), "prefix_len"),
        _ptr(tree_mask, torch.int64, (B, N, W), "tree_mask"), _ptr(n_nodes, torch.int32, (B,), "n_nodes"),
        B, N, Hq, Hkv, d, S_max, float(scale), code, _ptr(out, dt, (B, N, Hq, d), "out"),
        _ptr(lse, torch.float32, (B, N, Hq), "lse"), _ptr(err, torch.int32, (B,), "err"),
        _ptr(ws, None, None, "workspace"), ws.numel(), _stream(stream)), "spec_tree_attn")
    return {"out": out, "lse": lse, "err": err}


# ----------------------------------------------------------------------------- verify

def verify_workspace_bytes(B, N, V):
    return int(lib().spec_verify_workspace(B, N, V))


def spec_verify(target_logits, tokens, parents, uniforms, mode, draft_probs=None, draft_row=None,
                t2d=None, n_nodes=None, eps=0.09, delta=0.3, max_depth=None, out=None, ws=None,
                stream=None):
    B, N, V = target_logits.shape
    dev = target_logits.device
    mode = MODES.get(mode, mode)
    if max_depth is None:
        max_depth = N - 1
    R = Vd = 0
    if draft_probs is not None:
        _, R, Vd = draft_probs.shape
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(verify_workspace_bytes(B, N, V), dev)
    _check(lib().spec_verify(
        _ptr(target_logits, torch.float32, (B, N, V), "target_logits"),
        _ptr(draft_probs, torch.float32, (B, R, Vd), "draft_probs"),
        _ptr(draft_row, torch.int32, (B, N), "draft_row"), _ptr(t2d, torch.int32, (V,), "t2d"),
        _ptr(tokens, torch.int32, (B, N), "tokens"), _ptr(parents, torch.int32, (B, N), "parents"),
        _ptr(n_nodes, torch.int32, (B,), "n_nodes"), _ptr(uniforms, torch.float32, (B, N), "uniforms"),
        B, N, V, R, Vd, int(max_depth), int(mode), float(eps), float(delta),
        _ptr(out["accept_len"], torch.int32, (B,), "accept_len"),
        _ptr(out["path"], torch.int32, (B, max_depth + 1), "path"),
        _ptr(out["bonus"], torch.int32, (B,), "bonus"),
        _ptr(out["node_accept"], torch.uint8, (B, N), "node_accept"),
        _ptr(out["err"], torch.int32, (B,), "err"), _ptr(ws, None, None, "workspace"), ws.numel(),
        _stream(stream)), "spec_verify")
    return out


def verify_static_bytes(B, N, V):
    return int(lib().spec_verify_static_bytes(B, N, V))


def spec_verify_static(target_logits, tokens, parents, uniforms, mode, draft_probs=None, draft_row=None,
                       t2d=None, n_nodes=None, eps=0.09, delta=0.3, max_depth=None, out=None, stream=None):
    """spec_verify with the library's fixed scratch array instead of a workspace (no device
    allocation inside the call when ``out`` is given)."""
    B, N, V = target_logits.shape
    dev = target_logits.device
    mode = MODES.get(mode, mode)
    if max_depth is None:
        max_depth = N - 1
    R = Vd = 0
    if draft_probs is not None:
        _, R, Vd = draft_probs.shape
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib().spec_verify_static(
        _ptr(target_logits, torch.float32, (B, N, V), "target_logits"),
        _ptr(draft_probs, torch.float32, (B, R, Vd), "draft_probs"),
        _ptr(draft_row, torch.int32, (B, N), "draft_row"), _ptr(t2d, torch.int32, (V,), "t2d"),
        _ptr(tokens, torch.int32, (B, N), "tokens"), _ptr(parents, torch.int32, (B, N), "parents"),
        _ptr(n_nodes, torch.int32, (B,), "n_nodes"), _ptr(uniforms, torch.float32, (B, N), "uniforms"),
        B, N, V, R, Vd, int(max_depth), int(mode), float(eps), float(delta),
        _ptr(out["accept_len"], torch.int32, (B,), "accept_len"),
        _ptr(out["path"], torch.int32, (B, max_depth + 1), "path"),
        _ptr(out["bonus"], torch.int32, (B,), "bonus"),
        _ptr(out["node_accept"], torch.uint8, (B, N), "node_accept"),
        _ptr(out["err"], torch.int32, (B,), "err"), _stream(stream)), "spec_verify_static")
    return out


# ----------------------------------------------------------------------------- target LM head + row statistics

def lm_head_stats_workspace_bytes(B, N, Dm, V):
    return int(lib().spec_lm_head_stats_workspace(B, N, Dm, V))


def spec_lm_head_stats(hidden, W, parents, tokens, n_nodes=None, out=None, ws=None, stream=None):
    B, N, Dm = hidden.shape
    V = W.shape[0]
    dev = hidden.device
    if out is None:
        out = {"row_max": torch.empty((B, N), dtype=torch.float32, device=dev),
               "row_argmax": torch.empty((B, N), dtype=torch.int32, device=dev),
               "row_sum": torch.empty((B, N), dtype=torch.float64, device=dev),
               "row_ent": torch.empty((B, N), dtype=torch.float64, device=dev),
               "cand_logit": torch.empty((B, N), dtype=torch.float32, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(lm_head_stats_workspace_bytes(B, N, Dm, V), dev)
    _check(lib().spec_lm_head_stats(
        _ptr(hidden, torch.bfloat16, (B, N, Dm), "hidden"), _ptr(W, torch.bfloat16, (V, Dm), "W"),
        _ptr(parents, torch.int32, (B, N), "parents"), _ptr(tokens, torch.int32, (B, N), "tokens"),
        _ptr(n_nodes, torch.int32, (B,), "n_nodes"), B, N, Dm, V,
        _ptr(out["row_max"], torch.float32, (B, N), "row_max"),
        _ptr(out["row_argmax"], torch.int32, (B, N), "row_argmax"),
        _ptr(out["row_sum"], torch.float64, (B, N), "row_sum"),
        _ptr(out["row_ent"], torch.float64, (B, N), "row_ent"),
        _ptr(out["cand_logit"], torch.float32, (B, N), "cand_logit"),
        _ptr(out["err"], torch.int32, (B,), "err"), _ptr(ws, None, None, "workspace"), ws.numel(),
        _stream(stream)), "spec_lm_head_stats")
    return out


def spec_verify_greedy_stats(row_argmax, tokens, parents, V, n_nodes=None, max_depth=None, out=None, stream=None):
    B, N = tokens.shape
    dev = tokens.device
    if max_depth is None:
        max_depth = N - 1
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib().spec_verify_greedy_stats(
        _ptr(row_argmax, torch.int32, (B, N), "row_argmax"), _ptr(tokens, torch.int32, (B, N), "tokens"),
        _ptr(parents, torch.int32, (B, N), "parents"), _ptr(n_nodes, torch.int32, (B,), "n_nodes"),
        B, N, int(V), int(max_depth),
        _ptr(out["accept_len"], torch.int32, (B,), "accept_len"),
        _ptr(out["path"], torch.int32, (B, max_depth + 1), "path"),
        _ptr(out["bonus"], torch.int32, (B,), "bonus"),
        _ptr(out.get("node_accept"), torch.uint8, (B, N), "node_accept"),
        _ptr(out["err"], torch.int32, (B,), "err"), _stream(stream)), "spec_verify_greedy_stats")
    return out


def verify_lm_head_workspace_bytes(B, N, Dm, V, mode="typical"):
    return int(lib().spec_verify_lm_head_workspace(B, N, Dm, V, int(MODES.get(mode, mode))))


def spec_verify_lm_head(hidden, W, tokens, parents, uniforms, mode, n_nodes=None, draft_probs=None, draft_row=None,
                        t2d=None, eps=0.09, delta=0.3, max_depth=None, out=None, ws=None, stream=None):
    B, N, Dm = hidden.shape
    V = W.shape[0]
    R = Vd = 0
    if draft_probs is not None:
        _, R, Vd = draft_probs.shape
    dev = hidden.device
    mode = MODES.get(mode, mode)
    if max_depth is None:
        max_depth = N - 1
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
               "err": torch.empty((B,), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(verify_lm_head_workspace_bytes(B, N, Dm, V, mode), dev)
    _check(lib().spec_verify_lm_head(
        _ptr(hidden, torch.bfloat16, (B, N, Dm), "hidden"), _ptr(W, torch.bfloat16, (V, Dm), "W"),
        _ptr(tokens, torch.int32, (B, N), "tokens"), _ptr(parents, torch.int32, (B, N), "parents"),
        _ptr(n_nodes, torch.int32, (B,), "n_nodes"), _ptr(uniforms, torch.float32, (B, N), "uniforms"),
        _ptr(draft_probs, torch.float32, (B, R, Vd), "draft_probs"), _ptr(draft_row, torch.int32, (B, N), "draft_row"),
        _ptr(t2d, torch.int32, (V,), "t2d"), B, N, Dm, V, R, Vd, int(max_depth), int(mode), float(eps), float(delta),
        _ptr(out["accept_len"], torch.int32, (B,), "accept_len"),
        _ptr(out["path"], torch.int32, (B, max_depth + 1), "path"),
        _ptr(out["bonus"], torch.int32, (B,), "bonus"),
        _ptr(out.get("node_accept"), torch.uint8, (B, N), "node_accept"),
        _ptr(out["err"], torch.int32, (B,), "err"), _ptr(ws, None, None, "workspace"), ws.numel(),
        _stream(stream)), "spec_verify_lm_head")
    return out


# ----------------------------------------------------------------------------- heads

def medusa_heads_workspace_bytes(B, H, Dm, V, k):
    return int(lib().spec_medusa_heads_workspace(B, H, Dm, V, k))


def spec_medusa_heads(h, W_res, W_lm, k, out=None, want_probs=True, ws=None, stream=None):
    B, Dm = h.shape
    H = W_res.shape[0]
    V = W_lm.shape[0]
    dev = h.device
    if out is None:
        out = {"topk_idx": torch.empty((B, H, k), dtype=torch.int32, device=dev),
               "topk_prob": torch.empty((B, H, k), dtype=torch.float32, device=dev),
               "probs": torch.empty((B, H, V), dtype=torch.float32, device=dev) if want_probs else None}
    if ws is None:
        ws = workspace(medusa_heads_workspace_bytes(B, H, Dm, V, k), dev)
    _check(lib().spec_medusa_heads(
        _ptr(h, torch.bfloat16, (B, Dm), "h"), _ptr(W_res, torch.bfloat16, (H, Dm, Dm), "W_res"),
        _ptr(W_lm, torch.bfloat16, (V, Dm), "W_lm"), B, H, Dm, V, k,
        _ptr(out["topk_idx"], torch.int32, (B, H, k), "topk_idx"),
        _ptr(out["topk_prob"], torch.float32, (B, H, k), "topk_prob"),
        _ptr(out["probs"], torch.float32, (B, H, V), "probs"),
        _ptr(ws, None, None, "workspace"), ws.numel(), _stream(stream)), "spec_medusa_heads")
    return out


# ----------------------------------------------------------------------------- KV compaction

def spec_kv_compact(k_cache, v_cache, prefix_len, path, accept_len, err=None, prefix_len_out=None,
                    stream=None):
    """Compact the accepted path's K/V after the prefix, in place, in every layer.

    k_cache, v_cache: [L, B, Hkv, S_max, d] or [B, Hkv, S_max, d] (one layer), bf16 or f32,
    contiguous.  path / accept_len / err: spec_verify's outputs.  Returns the new prefix
    lengths (``prefix_len_out``, allocated when None; it must not be ``prefix_len``)."""
    if k_cache.dim() == 4:
        L, (B, Hkv, S_max, d) = 1, k_cache.shape
    else:
        L, B, Hkv, S_max, d = k_cache.shape
    dt = k_cache.dtype
    code = {torch.bfloat16: SPEC_BF16, torch.float32: SPEC_F32}.get(dt)
    if code is None:
        raise SpecError("k_cache must be bfloat16 or float32")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise SpecError("v_cache must have the shape of k_cache")
    max_depth = path.shape[1] - 1
    if prefix_len_out is None:
        prefix_len_out = torch.empty_like(prefix_len)
    _check(lib().spec_kv_compact(
        _ptr(k_cache, dt, None, "k_cache"), _ptr(v_cache, dt, None, "v_cache"), B * Hkv * S_max * d, L,
        _ptr(prefix_len, torch.int32, (B,), "prefix_len"),
        _ptr(prefix_len_out, torch.int32, (B,), "prefix_len_out"),
        _ptr(path, torch.int32, (B, max_depth + 1), "path"), _ptr(accept_len, torch.int32, (B,), "accept_len"),
        _ptr(err, torch.int32, (B,), "err"), B, Hkv, S_max, d, max_depth, code, _stream(stream)),
        "spec_kv_compact")
    return prefix_len_out


# ----------------------------------------------------------------------------- timing

def prof_enable(on=True):
    lib().spec_prof_enable(1 if on else 0)


def prof_reset():
    lib().spec_prof_reset()


def prof_read(name):
    """(total milliseconds, launches) recorded for kernel `name`, or (0.0, 0)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    lib().spec_prof_read(name.encode(), ctypes.byref(ms), ctypes.byref(n))
    return ms.value, n.value


def tune(name, value):
    """Force a launch-shape choice of the library (internal; tests cover every shape it can
    pick).  ``value`` None removes the override.  Results do not depend on it."""
    if lib().spec_internal_tune(name.encode(), -1 if value is None else int(value)) != 0:
        raise SpecError(f"unknown tuning override {name!r}")


class tuned:
    """Context manager: ``with tuned(attn_cb=2, attn_splits=3): ...`` forces those launch
    shapes inside the block and removes the overrides on exit."""

    def __init__(self, **knobs):
        self.knobs = knobs

    def __enter__(self):
        for k, v in self.knobs.items():
            tune(k, v)
        return self

    def __exit__(self, *exc):
        for k in self.knobs:
            tune(k, None)
        return False
