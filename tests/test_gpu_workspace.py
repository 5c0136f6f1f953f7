"""The header's workspace contract: a workspace needs no initialisation, and every output
element a call documents is written.  Each entry point runs twice on the same inputs, once
with every workspace and output byte set to 0x00 and once to 0xFF; the outputs must be
bit-identical.  A kernel that read a workspace byte it had not written in the same call (a
leaf row's partials, a stale plan, a list entry past its count), or left an output element
unwritten, would see different bytes in the two runs."""

import numpy as np
import pytest
import torch

from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import dev, need_gpu

pytestmark = pytest.mark.gpu


def _filled(tensors, fill):
    """Copies of the output tensors (a dict, or a list of tensors) with every byte = fill."""
    if isinstance(tensors, dict):
        return {k: _filled(v, fill) if v is not None else None for k, v in tensors.items()}
    t = torch.empty_like(tensors)
    t.view(torch.uint8).fill_(fill)
    return t


def _bits(x):
    if isinstance(x, dict):
        return {k: _bits(v) for k, v in x.items() if v is not None}
    return x.contiguous().view(torch.uint8).cpu().numpy().copy()


def _same(a, b, what):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: output {k} depends on the initial workspace/output bytes"


def _twice(call, ws_bytes, outs, what):
    """call(ws, out) with everything 0x00, then 0xFF; returns the first run's outputs."""
    need_gpu()
    res = []
    for fill in (0x00, 0xFF):
        ws = sb.workspace(ws_bytes, "cuda", fill=fill)
        out = _filled(outs, fill)
        call(ws, out)
        torch.cuda.synchronize()
        res.append(_bits(out))
    _same(res[0], res[1], what)
    print(f"{what}: {ws_bytes} workspace bytes, outputs identical under 0x00 / 0xFF fills", flush=True)
    return res[0]


def _tree(w):
    a = wl.attention_inputs(w)
    par, nn, P = dev(a["parents"]), dev(a["n_nodes"]), dev(a["prefix_len"])
    tb = sb.spec_tree_build(par, prefix_len=P, n_nodes=nn)
    return a, par, nn, P, tb


@pytest.mark.parametrize("splits", [None, 1, 3])
def test_tree_build_and_attention(tune, splits):
    w = wl.custom(seed=610, B=3, N=45, Hq=16, Hkv=4, d=128, prefix=("uniform", 1, 900), tree=("random", 5),
                  n_nodes_range=(20, 45), extra_slots=9)
    if splits is not None:
        tune(attn_splits=splits)
    a, par, nn, P, tb = _tree(w)
    _twice(lambda ws, out: sb.spec_tree_build(par, prefix_len=P, n_nodes=nn, out=out), 1, dict(tb), "tree_build")
    q, k, v = (dev(a[x], torch.bfloat16) for x in ("q", "k_cache", "v_cache"))
    need = sb.tree_attn_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.d, a["S_max"], torch.bfloat16)
    outs = {"out": torch.empty_like(q), "lse": torch.empty((w.B, w.N, w.Hq), device="cuda"),
            "err": torch.empty((w.B,), dtype=torch.int32, device="cuda")}
    _twice(lambda ws, o: sb.spec_tree_attn(q, k, v, P, tb["mask"], n_nodes=nn, scale=a["scale"], out=o["out"],
                                           lse=o["lse"], err=o["err"], ws=ws), need, outs, f"tree_attn splits={splits}")
    w1 = wl.config(1)
    a1, par1, nn1, P1, tb1 = _tree(w1)
    q1, k1, v1 = (dev(a1[x]) for x in ("q", "k_cache", "v_cache"))
    outs1 = {"out": torch.empty_like(q1), "lse": torch.empty((1, w1.N, w1.Hq), device="cuda"),
             "err": torch.empty((1,), dtype=torch.int32, device="cuda")}
    _twice(lambda ws, o: sb.spec_tree_attn(q1, k1, v1, P1, tb1["mask"], n_nodes=nn1, out=o["out"], lse=o["lse"],
                                           err=o["err"], ws=ws), 1, outs1, "tree_attn fp32")


VERIFY_CASES = [dict(B=5, N=63, V=9000, n_nodes_range=(1, 63), tree=("random", 5)),
                dict(B=3, N=130, V=4099, Vd=3000, tree=("random", 7)),
                dict(B=12, N=20, V=2048, n_nodes_range=(0, 20), tree=("random", 4))]


@pytest.mark.parametrize("case", range(len(VERIFY_CASES)))
@pytest.mark.parametrize("mode", ["greedy", "typical", "reject", "walk"])
@pytest.mark.parametrize("forced", [{}, {"verify_rows_list": 1, "verify_store_w": 0},
                                    {"verify_rows_list": 0, "verify_store_w": 1, "verify_chunk": 4096}])
def test_verify(tune, case, mode, forced):
    w = wl.custom(seed=620 + case, **VERIFY_CASES[case])
    tune(**forced)
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    rej = mode in ("reject", "walk")
    args = (dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents), dev(vi["uniforms"]), mode)
    kw = dict(draft_probs=dev(vi["draft_probs"]) if rej else None, draft_row=dev(vi["draft_row"]) if rej else None,
              t2d=dev(vi["t2d"]) if (rej and vi["t2d"] is not None) else None, n_nodes=dev(n_nodes))
    outs = sb.spec_verify(*args, **kw)
    _twice(lambda ws, o: sb.spec_verify(*args, **kw, out=o, ws=ws), sb.verify_workspace_bytes(w.B, w.N, w.V), outs,
           f"verify {mode} case {case} {forced}")


def test_medusa_heads_and_assembly():
    w = wl.custom(seed=630, B=5, V=3001, heads={"H": 3, "Dm": 384, "k": 6})
    hi = wl.heads_inputs(w)
    h, Wr, Wl = dev(hi["h"], torch.bfloat16), dev(hi["W_res"], torch.bfloat16), dev(hi["W_lm"], torch.bfloat16)
    outs = sb.spec_medusa_heads(h, Wr, Wl, hi["k"])
    first = _twice(lambda ws, o: sb.spec_medusa_heads(h, Wr, Wl, hi["k"], out=o, ws=ws),
                   sb.medusa_heads_workspace_bytes(w.B, 3, 384, w.V, 6), outs, "medusa_heads")
    topo = dev(wl.bfs_tree((6, 3, 2), 40))
    topk = outs["topk_idx"]
    asm = sb.spec_tree_assemble(topk, topo)
    _twice(lambda ws, o: sb.spec_tree_assemble(topk, topo, out=o), 1, asm, "tree_assemble")
    assert first["topk_idx"].size > 0


def test_tree_select():
    pool = wl.random_pool(seed=640, B=3, C=700)
    d = {k: dev(v) for k, v in pool.items()}
    outs = sb.spec_tree_select(d["cand_parents"], d["cand_prob"], 50, cand_tokens=d["cand_tokens"],
                               cand_row=d["cand_row"])
    _twice(lambda ws, o: sb.spec_tree_select(d["cand_parents"], d["cand_prob"], 50, cand_tokens=d["cand_tokens"],
                                             cand_row=d["cand_row"], out=o), 1, outs, "tree_select")


@pytest.mark.parametrize("mode", ["greedy", "typical", "reject", "walk"])
def test_lm_head(mode):
    inp = wl.lm_head_inputs(seed=650, B=3, N=24, Dm=256, V=3000, max_depth=5)
    h, W = dev(inp["hidden"], torch.bfloat16), dev(inp["W"], torch.bfloat16)
    par, tok = dev(inp["parents"]), dev(inp["tokens"])
    nn = dev(np.array([24, 7, 0], np.int32))
    st = sb.spec_lm_head_stats(h, W, par, tok, n_nodes=nn)
    _twice(lambda ws, o: sb.spec_lm_head_stats(h, W, par, tok, n_nodes=nn, out=o, ws=ws),
           sb.lm_head_stats_workspace_bytes(3, 24, 256, 3000), st, "lm_head_stats")
    g = np.random.default_rng(650)
    unif = dev(g.random((3, 24), dtype=np.float32))
    draft = drow = None
    if mode in ("reject", "walk"):
        dp = g.random((3, 24, 3000)).astype(np.float32)
        draft = dev(dp / dp.sum(axis=2, keepdims=True))
        drow = dev(np.maximum(inp["parents"], 0).astype(np.int32))
    outs = sb.spec_verify_lm_head(h, W, tok, par, unif, mode, n_nodes=nn, draft_probs=draft, draft_row=drow)
    _twice(lambda ws, o: sb.spec_verify_lm_head(h, W, tok, par, unif, mode, n_nodes=nn, draft_probs=draft,
                                                draft_row=drow, out=o, ws=ws),
           sb.verify_lm_head_workspace_bytes(3, 24, 256, 3000, mode), outs, f"verify_lm_head {mode}")
    if mode == "greedy":
        g_outs = sb.spec_verify_greedy_stats(st["row_argmax"], tok, par, 3000, n_nodes=nn)
        _twice(lambda ws, o: sb.spec_verify_greedy_stats(st["row_argmax"], tok, par, 3000, n_nodes=nn, out=o), 1,
               g_outs, "verify_greedy_stats")


@pytest.mark.parametrize("Vd,mapped", [(20000, True), (777, False)])
def test_assemble_rows(Vd, mapped):
    w = wl.custom(seed=660, B=4, N=50, V=3 * Vd if mapped else Vd, Vd=Vd if mapped else None, tree=("random", 5),
                  n_nodes_range=(0, 50))
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    draft, par, row, nn = dev(vi["draft_probs"]), dev(parents), dev(vi["draft_row"]), dev(n_nodes)
    d2t = dev(vi["d2t"]) if vi["d2t"] is not None else None
    outs = sb.spec_tree_assemble_rows(draft, par, row, d2t=d2t, V=w.V, n_nodes=nn)
    _twice(lambda ws, o: sb.spec_tree_assemble_rows(draft, par, row, d2t=d2t, V=w.V, n_nodes=nn, out=o, ws=ws),
           sb.tree_assemble_rows_workspace_bytes(4, 50, Vd), outs, f"tree_assemble_rows Vd={Vd}")
