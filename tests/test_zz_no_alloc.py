"""spec_verify_static (verification with the library's fixed scratch array, no allocation)
against spec_verify (the same kernels with a caller workspace): outputs must be identical, on
two calls in a row, the second with a smaller input, and both must match the oracle.  The
scratch array keeps the first call's contents when the second runs."""

import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import compare_verify, dev, host, need_gpu

pytestmark = pytest.mark.gpu

MODE = {"greedy": oracle.MODE_GREEDY, "typical": oracle.MODE_TYPICAL, "reject": oracle.MODE_REJECT,
        "walk": oracle.MODE_WALK}


def _inputs(w):
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    return parents, n_nodes, vi


def _both(w, mode, parents, n_nodes, vi):
    rej = mode in ("reject", "walk")
    args = (dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents.astype(np.int32)), dev(vi["uniforms"]), mode)
    kw = dict(draft_probs=dev(vi["draft_probs"]) if rej else None, draft_row=dev(vi["draft_row"]) if rej else None,
              t2d=dev(vi["t2d"]) if (rej and vi["t2d"] is not None) else None,
              n_nodes=dev(n_nodes.astype(np.int32)), eps=float(np.float32(0.09)), delta=float(np.float32(0.3)))
    print(f"spec_verify_static {w.name}: B={w.B} N={w.N} V={w.V} mode={mode}, "
          f"{sb.verify_static_bytes(w.B, w.N, w.V)} scratch bytes", flush=True)
    st = sb.spec_verify_static(*args, **kw)
    ws = sb.spec_verify(*args, **kw, ws=sb.workspace(sb.verify_workspace_bytes(w.B, w.N, w.V), "cuda", fill=0xFF))
    torch.cuda.synchronize()
    st = {k: host(v) for k, v in st.items()}
    ws = {k: host(v) for k, v in ws.items()}
    for k in ws:
        assert np.array_equal(st[k], ws[k]), f"{w.name} {mode}: {k} differs from spec_verify"
    ref = oracle.verify(vi["target_logits"], vi["tokens"], parents, vi["uniforms"], MODE[mode],
                        draft_probs=vi["draft_probs"], draft_row=vi["draft_row"], t2d=vi["t2d"], n_nodes=n_nodes,
                        eps=float(np.float32(0.09)), delta=float(np.float32(0.3)))
    compare_verify(st, ref, n_nodes, walk=mode == "walk", bonus_margin=1e-7 if mode == "walk" else 1e-9)
    return st


def test_static_scratch_matches_workspace_twice():
    need_gpu()
    big = wl.config(3)                         # 16 x 127 nodes, vocabulary 128256: ~3.6 MB of scratch
    small = wl.custom(seed=901, B=3, N=37, V=5000, tree=("random", 5), n_nodes_range=(20, 37))
    assert sb.verify_static_bytes(small.B, small.N, small.V) < sb.verify_static_bytes(big.B, big.N, big.V)
    _both(big, "reject", *_inputs(big))
    _both(small, "typical", *_inputs(small))
    _both(small, "walk", *_inputs(small))


def test_static_scratch_limit():
    """A request beyond the array is refused on the host (nothing is launched)."""
    need_gpu()
    B, N, V = 8, 256, 1_000_000
    assert sb.verify_static_bytes(B, N, V) > 16 << 20
    t = torch.zeros((1,), device="cuda")
    L = sb.lib()
    fake = t.data_ptr()
    st = L.spec_verify_static(fake, None, None, None, fake, fake, None, fake, B, N, V, 0, 0, N - 1, 0, 0.1, 0.3,
                              fake, fake, fake, None, fake, None)
    assert st == 5 and L.spec_strerror(st).decode() == "request exceeds the fixed scratch array"
