#!/usr/bin/env python3
"""One-GPU benchmark of the tree-verification step of Medusa/EAGLE-style speculative decoding.

A step is one pass of every hot-path stage the workload defines, on one batch of synthetic
input already resident in HBM:
    [Medusa-head workload only: heads -> tree assembly ->] tree build -> tree attention -> verify
(the 63/127/255-node workloads start from a drafted tree whose tokens are given; their
EAGLE-style assembly from the draft rows is timed beside the step, under next_rows)
The default workload is the 63-node Llama-3-8B-shaped one (batch 1, 32 query / 8 key-value
heads, head_dim 128, prefix 2048, vocabulary 128256, rejection-sampling verify).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Timing: W warm-up steps, then exactly K steps replayed from HIP graphs (one graph per cycle
over rotating input copies totalling more than 1 GB, so the 256 MB Infinity Cache cannot serve
repeats), bracketed by torch.cuda.synchronize() and HIP events.  A second pass over the same K
steps, launched eagerly with the library's kernel timing on (start/stop events stamped by each
kernel's own dispatch), gives each kernel's average launch duration for the roofline figure.  The CPU oracle is then timed on the host on a
bounded sample of the same workload.  Prints one JSON line on stdout; details go to stderr.
"""

import argparse
import json
import math
import os
import sys
import time

METRIC = "tree-verify nodes/s + % HBM roofline (63/127-node tree, 8B-shaped GQA)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 1-5 (default 2: 63-node tree)")
    ap.add_argument("--also", type=int, nargs="*", default=None,
                    help="further workloads timed into the same line (default: the 127-node batch-16 one "
                         "beside the 63-node default)")
    ap.add_argument("--mode", default=None, help="verify mode (default: the workload's last listed)")
    ap.add_argument("--rotate-gb", type=float, default=1.2, help="total size of rotating input copies")
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of from HIP graphs")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this size (for scaling --pmc byte counters)")
    ap.add_argument("--side-rows", action="store_true",
                    help="time the rows beside the step also in a counter run (--copy-calibration-mb)")
    args = ap.parse_args()
    if args.also is None:
        args.also = [3] if args.config == 2 and not args.copy_calibration_mb else []
    return args


# --------------------------------------------------------------------------- inputs

def host_inputs(w):
    from tree_attention_verification_spec_amd import workloads as wl
    a = wl.attention_inputs(w)
    if w.heads:
        return a, None, wl.heads_inputs(w), wl.heads_target_inputs(w)
    return a, wl.verify_inputs(w, a["parents"]), None, None


def upload(w, a, vi, hi, ti):
    import numpy as np
    import torch
    from tree_attention_verification_spec_amd import workloads as wl
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(x, dt=None):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.to(dt) if dt is not None else t).cuda()

    s = {"q": dev(a["q"], tdt), "k": dev(a["k_cache"], tdt), "v": dev(a["v_cache"], tdt),
         "P": dev(a["prefix_len"]), "parents": dev(a["parents"]), "n_nodes": dev(a["n_nodes"])}
    if w.heads:
        s.update(h=dev(hi["h"], torch.bfloat16), W_res=dev(hi["W_res"], torch.bfloat16),
                 W_lm=dev(hi["W_lm"], torch.bfloat16), topo=dev(wl.bfs_tree(w.tree[1], w.N)),
                 logits=dev(ti["target_logits"]), uniforms=dev(ti["uniforms"]))
    else:
        s.update(logits=dev(vi["target_logits"]), uniforms=dev(vi["uniforms"]), tokens=dev(vi["tokens"]),
                 draft=dev(vi["draft_probs"]), draft_row=dev(vi["draft_row"]))
        if vi["t2d"] is not None:
            s["t2d"] = dev(vi["t2d"])
            s["d2t"] = dev(vi["d2t"])
    return s


def set_bytes(s):
    return sum(t.numel() * t.element_size() for t in s.values())


def alloc_outputs(w, s):
    import torch
    B, N = w.B, w.N
    W = (N + 63) // 64
    o = {"tb": {"mask": torch.empty((B, N, W), dtype=torch.int64, device="cuda"),
                "positions": torch.empty((B, N), dtype=torch.int32, device="cuda"),
                "depths": torch.empty((B, N), dtype=torch.int32, device="cuda"),
                "err": torch.empty((B,), dtype=torch.int32, device="cuda")},
         "attn_out": torch.empty_like(s["q"]),
         "lse": torch.empty((B, N, w.Hq), dtype=torch.float32, device="cuda"),
         "attn_err": torch.empty((B,), dtype=torch.int32, device="cuda"),
         "ver": {"accept_len": torch.empty((B,), dtype=torch.int32, device="cuda"),
                 "path": torch.empty((B, N), dtype=torch.int32, device="cuda"),
                 "bonus": torch.empty((B,), dtype=torch.int32, device="cuda"),
                 "node_accept": torch.empty((B, N), dtype=torch.uint8, device="cuda"),
                 "err": torch.empty((B,), dtype=torch.int32, device="cuda")}}
    if w.heads:
        H, k, V = w.heads["H"], w.heads["k"], w.V
        o["heads"] = {"topk_idx": torch.empty((B, H, k), dtype=torch.int32, device="cuda"),
                      "topk_prob": torch.empty((B, H, k), dtype=torch.float32, device="cuda"),
                      "probs": torch.empty((B, H, V), dtype=torch.float32, device="cuda")}
        o["asm"] = {"tokens": torch.empty((B, N), dtype=torch.int32, device="cuda"),
                    "draft_row": torch.empty((B, N), dtype=torch.int32, device="cuda"),
                    "err": torch.empty((B,), dtype=torch.int32, device="cuda")}
    return o


# --------------------------------------------------------------------------- one step

class Stepper:
    def __init__(self, w, mode, sets):
        import torch
        from tree_attention_verification_spec_amd import binding as sb
        self.w, self.mode, self.sets, self.sb = w, mode, sets, sb
        self.outs = [alloc_outputs(w, s) for s in sets]
        s0 = sets[0]
        B, N, Hq, Hkv, d = w.B, w.N, w.Hq, w.Hkv, w.d
        S_max = s0["k"].shape[2]
        self.ws_attn = sb.workspace(sb.tree_attn_workspace_bytes(B, N, Hq, Hkv, d, S_max, s0["q"].dtype), "cuda")
        self.ws_ver = sb.workspace(sb.verify_workspace_bytes(B, N, w.V), "cuda")
        if w.heads:
            self.ws_heads = sb.workspace(sb.medusa_heads_workspace_bytes(B, w.heads["H"], w.heads["Dm"], w.V,
                                                                         w.heads["k"]), "cuda")

        self.scale = d ** -0.5

    def step(self, i):
        sb, w = self.sb, self.w
        s, o = self.sets[i], self.outs[i]
        if w.heads:
            sb.spec_medusa_heads(s["h"], s["W_res"], s["W_lm"], w.heads["k"], out=o["heads"], ws=self.ws_heads)
            sb.spec_tree_assemble(o["heads"]["topk_idx"], s["topo"], out=o["asm"])
            tokens, draft, draft_row = o["asm"]["tokens"], o["heads"]["probs"], o["asm"]["draft_row"]
        else:
            tokens, draft, draft_row = s["tokens"], s["draft"], s["draft_row"]
        sb.spec_tree_build(s["parents"], prefix_len=s["P"], n_nodes=s["n_nodes"], out=o["tb"])
        sb.spec_tree_attn(s["q"], s["k"], s["v"], s["P"], o["tb"]["mask"], n_nodes=s["n_nodes"], scale=self.scale,
                          out=o["attn_out"], lse=o["lse"], err=o["attn_err"], ws=self.ws_attn)
        rej = self.mode in ("reject", "walk")
        sb.spec_verify(s["logits"], tokens, s["parents"], s["uniforms"], self.mode,
                       draft_probs=draft if rej else None, draft_row=draft_row if rej else None,
                       t2d=s.get("t2d") if rej else None, n_nodes=s["n_nodes"], max_depth=w.N - 1,
                       out=o["ver"], ws=self.ws_ver)


def capture(stepper, indices):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in indices:
            stepper.step(i)
    return g


# --------------------------------------------------------------------------- algorithmic work

def algorithmic(w, a, parents, depths, mode):
    """Per-launch algorithmic bytes / FLOPs of each kernel (what the method must move or do)."""
    import numpy as np
    s = 2 if w.dtype == "bf16" else 4
    B, N, Hq, Hkv, d, V = w.B, w.N, w.Hq, w.Hkv, w.d, w.V
    P = a["prefix_len"].astype(np.int64)
    n = a["n_nodes"].astype(np.int64)
    W = (N + 63) // 64
    attn_bytes = int(((P + n) * Hkv * d * 2 * s).sum() + 2 * B * N * Hq * d * s + B * N * W * 8)
    attn_flops = 0
    internal = branching = 0
    for b in range(B):
        nb = int(n[b])
        attn_flops += 4 * Hq * d * int((P[b] + depths[b, :nb] + 1).sum())
        kids = np.bincount(parents[b, 1:nb].clip(min=0), minlength=N)
        internal += int((kids > 0).sum())
        branching += int((kids > 1).sum())
    # the bonus pass reads the kept row once more, and a residual draw the draft row beside it
    kept = B * V * 4 * (2 if mode in ("reject", "walk") else 1)

    out = {("tree_attn_bf16" if w.dtype == "bf16" else "tree_attn_f32"): (attn_bytes, attn_flops),
           "verify_rows": (internal * V * 4, 0),
           "verify_decide_bonus": (kept, 0)}
    if mode == "walk":
        # the walk's residual chains: each node with two or more children reads its logits row
        # and its children's draft row once (the passes after the first are served by the caches)
        Vd = w.Vd or V
        out["verify_walk_chain"] = (branching * (V + Vd) * 4, 0)
    if w.heads:
        H, Dm = w.heads["H"], w.heads["Dm"]
        out["medusa_resblock"] = (H * Dm * Dm * 2, 2 * B * H * Dm * Dm)
        out["medusa_lm_head"] = (V * Dm * 2, 2 * B * H * Dm * V)
    return out


def kv_compact_timing(st, layers_max=32, cap_bytes=8 << 30, reps=50):
    """The KV-cache compaction that closes a round (a row after the verification step, measured
    outside it): a cache of the workload's KV shape with up to `layers_max` layers (32 for a
    Llama-3-8B-class model; fewer when the cache would pass `cap_bytes`), compacted with the
    step's own verification outputs.  The cache contents do not matter to the copy's time."""
    import torch
    from tree_attention_verification_spec_amd import binding as sb
    s0, ver = st.sets[0], st.outs[0]["ver"]
    B, Hkv, S_max, d = s0["k"].shape
    per_layer = 2 * B * Hkv * S_max * d * s0["k"].element_size()
    layers = int(max(1, min(layers_max, cap_bytes // per_layer)))
    k = torch.empty((layers, B, Hkv, S_max, d), dtype=s0["k"].dtype, device="cuda")
    v = torch.empty_like(k)
    P_out = torch.empty_like(s0["P"])
    call = lambda: sb.spec_kv_compact(k, v, s0["P"], ver["path"], ver["accept_len"], err=ver["err"],
                                      prefix_len_out=P_out)
    call()
    torch.cuda.synchronize()
    try:
        sb.prof_reset()
        sb.prof_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        sb.prof_enable(False)
        ms, cnt = sb.prof_read("kv_compact")
    finally:
        sb.prof_enable(False)
        sb.prof_reset()
    acc, err = ver["accept_len"].cpu().numpy(), ver["err"].cpu().numpy()
    rows = int(acc[err == 0].clip(min=0).sum())
    nbytes = 2 * rows * Hkv * d * k.element_size() * 2 * layers     # read + write, K and V
    del k, v
    us = ms / cnt * 1e3
    return {"layers": layers, "us": round(us, 3), "algorithmic_bytes": nbytes,
            "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 2) if us > 0 else None}


def assemble_rows_timing(st, reps=50):
    """EAGLE-style tree assembly (a row before the step, measured outside it): the workload's
    own tree and draft rows, each node's children taking the top candidates of their row; the
    tokens must equal the ones the step verifies."""
    import torch
    from tree_attention_verification_spec_amd import binding as sb
    w, s0 = st.w, st.sets[0]
    B, N = w.B, w.N
    Vd = s0["draft"].shape[2]
    ws = sb.workspace(sb.tree_assemble_rows_workspace_bytes(B, N, Vd), "cuda")
    call = lambda out=None: sb.spec_tree_assemble_rows(s0["draft"], s0["parents"], s0["draft_row"], d2t=s0.get("d2t"),
                                                        V=w.V, n_nodes=s0["n_nodes"], out=out, ws=ws)
    out = call()
    torch.cuda.synchronize()
    assert int(out["err"].abs().sum()) == 0
    assert torch.equal(out["tokens"][:, 1:], s0["tokens"][:, 1:]), "assembled tokens differ from the step's"
    try:
        sb.prof_reset()
        sb.prof_enable(True)
        for _ in range(reps):
            call(out)
        torch.cuda.synchronize()
        sb.prof_enable(False)
        ms1, c1 = sb.prof_read("assemble_chunks")
        ms2, c2 = sb.prof_read("assemble_merge")
        ms0, c0 = sb.prof_read("assemble_list")     # large grids list the nodes with children first
    finally:
        sb.prof_enable(False)
        sb.prof_reset()
    parents = s0["parents"].cpu()
    internal = sum(int(torch.unique(parents[b, 1:]).numel()) for b in range(B))
    nbytes = internal * Vd * 4
    us1, us2 = ms1 / c1 * 1e3, ms2 / c2 * 1e3
    us0 = ms0 / c0 * 1e3 if c0 else 0.0
    return {"shape": f"B{B} x {internal // B}-ish nodes with children x Vd {Vd}", "list_us": round(us0, 3),
            "chunks_us": round(us1, 3), "merge_us": round(us2, 3), "algorithmic_bytes": nbytes,
            "chunks_GBs": round(nbytes / (us1 * 1e-6) / 1e9, 1)}


def tree_select_timing(w, C=1024, reps=50):
    """Dynamic tree selection (a row before the step, measured outside it): per sequence of the
    workload's batch, a seeded pool of C drafted candidates (depth < 8) is cut to the workload's
    tree size."""
    import torch
    from tree_attention_verification_spec_amd import binding as sb
    from tree_attention_verification_spec_amd import workloads as wl
    pool = wl.random_pool(seed=5, B=w.B, C=C)
    d = {k: torch.from_numpy(v).cuda() for k, v in pool.items()}
    out = None
    call = lambda: sb.spec_tree_select(d["cand_parents"], d["cand_prob"], w.N, cand_tokens=d["cand_tokens"],
                                       cand_row=d["cand_row"], out=out)
    out = call()
    torch.cuda.synchronize()
    assert int(out["err"].abs().sum()) == 0
    try:
        sb.prof_reset()
        sb.prof_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        sb.prof_enable(False)
        ms, cnt = sb.prof_read("tree_select")
    finally:
        sb.prof_enable(False)
        sb.prof_reset()
    return {"pool": f"B{w.B} x {C} candidates -> {w.N} nodes", "us": round(ms / cnt * 1e3, 3)}


def lm_head_stats_timing(w, reps=20, Dm=4096):
    """The target LM head fused with the row statistics (a row beside the step, measured outside
    it) at the workload's batch and tree size (B * N <= 4096): hidden 4096, the workload's
    vocabulary.  Seeded random device inputs (their values do not change the time)."""
    import numpy as np
    import torch
    from tree_attention_verification_spec_amd import binding as sb
    from tree_attention_verification_spec_amd import workloads as wl
    B, N, V = w.B, w.N, w.V
    if B * N > 4096 or w.dtype != "bf16":
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    h = torch.randn((B, N, Dm), generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn((V, Dm), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    par = torch.from_numpy(np.stack(wl.trees(w)[0])).to(torch.int32).cuda()
    tok = torch.randint(0, V, (B, N), generator=g, device="cuda", dtype=torch.int32)
    out = sb.spec_lm_head_stats(h, W, par, tok)
    ver = sb.spec_verify_greedy_stats(out["row_argmax"], tok, par, V)
    uni = torch.rand((B, N), generator=g, device="cuda")
    vtyp = sb.spec_verify_lm_head(h, W, tok, par, uni, "typical")
    # draft rows that put most of their mass on the drafted tokens: the root's children are
    # rejected, so the residual draw takes the recomputed-row path (the costly case)
    drow = par.clamp(min=0)
    draft = torch.rand((B, N, V), generator=g, device="cuda") ** 8
    bi = torch.arange(B, device="cuda").unsqueeze(1).expand(B, N)
    draft[bi[:, 1:], drow[:, 1:].long(), tok[:, 1:].long()] += 1e4
    draft /= draft.sum(dim=2, keepdim=True)
    vrej = sb.spec_verify_lm_head(h, W, tok, par, uni, "reject", draft_probs=draft, draft_row=drow)
    vwalk = sb.spec_verify_lm_head(h, W, tok, par, uni, "walk", draft_probs=draft, draft_row=drow)
    torch.cuda.synchronize()
    assert int(out["err"].abs().sum()) == 0 and int(ver["err"].abs().sum()) == 0
    assert int(vtyp["err"].abs().sum()) == 0 and int(vrej["err"].abs().sum()) == 0
    assert int(vwalk["err"].abs().sum()) == 0
    try:
        sb.prof_reset()
        sb.prof_enable(True)
        for _ in range(reps):
            sb.spec_lm_head_stats(h, W, par, tok, out=out)
            sb.spec_verify_greedy_stats(out["row_argmax"], tok, par, V, out=ver)
        torch.cuda.synchronize()
        ms, cnt = sb.prof_read("lm_head_stats")
        ms2, cnt2 = sb.prof_read("lm_head_merge")
        ms3, cnt3 = sb.prof_read("lm_head_xperm")
        ms4, cnt4 = sb.prof_read("verify_greedy_stats")
        for _ in range(reps):
            sb.spec_verify_lm_head(h, W, tok, par, uni, "typical", out=vtyp)
        torch.cuda.synchronize()
        ms5, cnt5 = sb.prof_read("verify_lm")
        sb.prof_reset()
        for _ in range(reps):
            sb.spec_verify_lm_head(h, W, tok, par, uni, "reject", draft_probs=draft, draft_row=drow, out=vrej)
        torch.cuda.synchronize()
        sb.prof_enable(False)
        rej = [sb.prof_read(k) for k in ("verify_lm", "verify_lm_tilesum", "verify_lm_residual", "lm_head_stats")]
        sb.prof_reset()
        sb.prof_enable(True)
        for _ in range(reps):
            sb.spec_verify_lm_head(h, W, tok, par, uni, "walk", draft_probs=draft, draft_row=drow, out=vwalk)
        torch.cuda.synchronize()
        sb.prof_enable(False)
        wk_names = ("lm_head_stats", "verify_rows", "verify_rows_list", "verify_walk_chain", "verify_decide_bonus",
                    "verify_select")
        walk = {k: sb.prof_read(k) for k in wk_names}
    finally:
        sb.prof_enable(False)
        sb.prof_reset()
    us, us_merge, us_perm, us_greedy = ms / cnt * 1e3, ms2 / cnt2 * 1e3, ms3 / cnt3 * 1e3, ms4 / cnt4 * 1e3
    us_typ = ms5 / cnt5 * 1e3
    us_rej = [m / c * 1e3 for m, c in rej]
    us_walk = {("stats_with_rows" if k == "lm_head_stats" else k): round(m / c * 1e3, 3)
               for k, (m, c) in walk.items() if c}
    nbytes = V * Dm * 2 + B * N * Dm * 2
    flops = 2 * B * N * Dm * V
    del W, draft
    return {"shape": f"[{B * N} x {Dm}] x [{Dm} x {V}]", "us": round(us, 3), "merge_us": round(us_merge, 3),
            "xperm_us": round(us_perm, 3), "greedy_verify_us": round(us_greedy, 3),
            "typical_verify_us": round(us_typ, 3),
            "walk_verify_us": us_walk,
            "reject_verify_us": {"stats_with_rows": round(us_rej[3], 3), "decide": round(us_rej[0], 3),
                                 "tile_sums": round(us_rej[1], 3),
                                 "residual": round(us_rej[2], 3)},
            "algorithmic_bytes": nbytes, "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 8e12, 4),
            "achieved_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1)}


def roofline_entry(name, nbytes, flops, avg_ms, traffic):
    intensity = flops / nbytes if nbytes else 0.0
    if name.startswith("tree_attn") and intensity > RIDGE:
        achieved = flops / (avg_ms * 1e-3) / 1e12
        peak, unit, bound = BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved = nbytes / (avg_ms * 1e-3) / 1e9
        peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": name,
            "avg_us": round(avg_ms * 1e3, 3), "algorithmic_bytes": nbytes, "algorithmic_flops": flops}


# --------------------------------------------------------------------------- CPU oracle

def cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, a, vi, hi, ti, mode, budget_s, threads):
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from tree_attention_verification_spec_amd import workloads as wl
    modes = {"greedy": oracle.MODE_GREEDY, "typical": oracle.MODE_TYPICAL, "reject": oracle.MODE_REJECT,
             "walk": oracle.MODE_WALK}

    def one_round(ns):
        par = a["parents"][:1, :ns]
        P = a["prefix_len"][:1]
        nn = np.array([min(ns, int(a["n_nodes"][0]))])
        if w.heads:
            rh = oracle.medusa_heads(hi["h"][:1], hi["W_res"], hi["W_lm"], hi["k"])
            ra = oracle.tree_assemble(rh["topk_idx"], wl.bfs_tree(w.tree[1], w.N)[:ns])
            tokens, draft, drow, t2d = ra["tokens"], rh["probs"], ra["draft_row"], None
            logits, unif = ti["target_logits"][:1, :ns], ti["uniforms"][:1, :ns]
        else:
            tokens, draft, drow, t2d = vi["tokens"][:1, :ns], vi["draft_probs"][:1], vi["draft_row"][:1, :ns], vi["t2d"]
            logits, unif = vi["target_logits"][:1, :ns], vi["uniforms"][:1, :ns]
        tb = oracle.tree_build(par, nn, prefix_len=P)
        oracle.tree_attention(a["q"][:1, :ns], a["k_cache"][:1], a["v_cache"][:1], P, tb["dense"], nn, scale=a["scale"])
        oracle.verify(logits, tokens, par, unif, modes[mode], draft_probs=draft, draft_row=drow, t2d=t2d,
                      n_nodes=nn, max_depth=ns - 1)

    with threadpool_limits(threads):
        # size the sample from two probe rounds (1 and 2 nodes): fixed cost + cost per node
        t0 = time.perf_counter()
        one_round(1)
        t1 = time.perf_counter()
        one_round(min(2, w.N))
        t2 = time.perf_counter()
        per_node = max(t2 - t1 - (t1 - t0), 1e-4)
        fixed = max(t1 - t0 - per_node, 0.0)
        ns = int(max(1, min(w.N, (budget_s / 2.0 - fixed) / per_node)))
        rounds, start = 0, time.perf_counter()
        while True:
            one_round(ns)
            rounds += 1
            el = time.perf_counter() - start
            if el >= budget_s / 2.0 or rounds >= 50:
                break
    value = rounds * ns / el
    return {"value": round(value, 3), "unit": "tree-nodes/s", "cores": threads, "kind": "oracle",
            "sample": (f"sequence 0 of '{w.name}': first {ns} of {w.N} tree nodes, full prefix "
                       f"{int(a['prefix_len'][0])}; {rounds} oracle round(s) of "
                       f"{'heads + assembly + ' if w.heads else ''}tree build + attention over all "
                       f"{ns}x{w.Hq} query rows + {mode} verify; NumPy float64, {threads} BLAS thread(s); "
                       f"{el:.1f} s"),
            "host_cpus": os.cpu_count(), "host_cpu_model": cpu_model()}


# --------------------------------------------------------------------------- main

def measure(args, cfg, K, warmup, side, log_prefix=""):
    """Time K steps of workload `cfg` (graph replays over rotating input copies), then the
    per-kernel durations, the rows beside the step (when `side`), and the roofline entry."""
    import numpy as np
    import torch
    from tree_attention_verification_spec_amd import binding as sb
    from tree_attention_verification_spec_amd import profiling
    from tree_attention_verification_spec_amd import workloads as wl

    w = wl.config(cfg)
    mode = (args.mode if cfg == args.config else None) or w.modes[-1]
    log(f"{log_prefix}workload: {w.name}; verify mode {mode}")
    t0 = time.time()
    a, vi, hi, ti = host_inputs(w)
    base = upload(w, a, vi, hi, ti)
    per_set = set_bytes(base)
    nsets = max(2, math.ceil(args.rotate_gb * 1e9 / per_set))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    log(f"inputs: {per_set / 1e6:.1f} MB per copy x {nsets} rotating copies ({time.time() - t0:.1f} s)")
    st = Stepper(w, mode, sets)

    # eager warm-up and a reference result for the graph check
    for i in range(warmup):
        st.step(i % nsets)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in st.outs[0]["ver"].items()}
    ref_attn = st.outs[0]["attn_out"].clone()

    use_graph = not args.no_graph
    if use_graph:
        cyc = capture(st, range(nsets))
        rem = K % nsets
        rem_g = capture(st, range(rem)) if rem else None
        reps = K // nsets

        def run_k():
            for _ in range(reps):
                cyc.replay()
            if rem_g is not None:
                rem_g.replay()
        run_k()   # warm the graphs
        torch.cuda.synchronize()
        for k, v in st.outs[0]["ver"].items():
            assert torch.equal(v, ref[k]), f"graph replay differs from eager ({k})"
        assert torch.equal(st.outs[0]["attn_out"], ref_attn), "graph replay differs from eager (attention)"
    else:
        def run_k():
            for i in range(K):
                st.step(i % nsets)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run_k()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    err_words = torch.cat([st.outs[0]["ver"]["err"], st.outs[0]["attn_err"], st.outs[0]["tb"]["err"]])
    assert int(err_words.abs().sum()) == 0, "a sequence reported a data error"

    # per-kernel durations: the same K steps launched eagerly with the library's kernel timing
    # on (each launch carries a start/stop event pair stamped by its own dispatch)
    names = ("tree_build", "tree_assemble", "tree_attn_bf16", "tree_attn_merge", "tree_attn_f32", "verify_rows_list",
             "verify_rows", "verify_walk_chain", "verify_decide_bonus", "verify_select", "medusa_resblock",
             "medusa_lm_head", "medusa_softmax_topk")
    kernels = {}
    try:
        sb.prof_reset()
        sb.prof_enable(True)
        torch.cuda.synchronize()
        for i in range(K):
            st.step(i % nsets)
        torch.cuda.synchronize()
        sb.prof_enable(False)
        for name in names:
            ms, cnt = sb.prof_read(name)
            if cnt:
                kernels[name] = ms / cnt
    finally:
        sb.prof_enable(False)
        sb.prof_reset()

    depths = st.outs[0]["tb"]["depths"].cpu().numpy()
    accept_mean = float(st.outs[0]["ver"]["accept_len"].float().mean().item())
    work = algorithmic(w, a, a["parents"], depths, mode)
    # the dominant kernel: the longest on average; kernels within 3 % of it count as tied (at
    # batch 1 attention and the decision kernel differ by less than their run-to-run spread),
    # and a tie goes to the one that moves the most algorithmic bytes
    longest = max(kernels[k] for k in kernels if k in work)
    dom = max((k for k in kernels if k in work and kernels[k] >= 0.97 * longest), key=lambda k: work[k][0])
    nbytes, flops = work[dom]
    # every kernel with an algorithmic figure against its own bound (HBM, or the bf16 MFMA peak
    # for attention above the ridge)
    kernels_frac = {k: roofline_entry(k, *work[k], kernels[k], None)["frac"] for k in kernels if k in work}
    short = {1: "tiny", 2: "tree63", 3: "tree127_b16", 4: "tree255_b4", 5: "medusa_tree127_b8"}[cfg]
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{dom}_{short}.md"))
    roof = roofline_entry(dom, nbytes, flops, kernels[dom], None if tr is None else int(tr[0]))
    for k in sorted(kernels, key=lambda k: -kernels[k]):
        extra = ""
        if k in work:
            b_, f_ = work[k]
            extra = f"  {b_ / (kernels[k] * 1e-3) / 1e9:8.1f} GB/s  {f_ / (kernels[k] * 1e-3) / 1e12:8.1f} TFLOP/s"
        log(f"  {k:22s} {kernels[k] * 1e3:9.2f} us{extra}")
    log(f"step {ms_step * 1e3:.2f} us; kernels sum {sum(kernels.values()) * 1e3:.2f} us")
    # the whole step against the HBM roofline: every kernel's algorithmic bytes in one step
    step_bytes = sum(b_ for b_, _ in work.values())
    step_flops = sum(f_ for _, f_ in work.values())
    step_roof = {"algorithmic_bytes": step_bytes, "algorithmic_flops": step_flops,
                 "hbm_frac": round(step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                 "bound_us": round(max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e6, 3)}
    log(f"step: {step_bytes / 1e6:.1f} MB algorithmic, {step_roof['hbm_frac'] * 100:.1f} % of the HBM roofline")
    # the rows beside the step; skipped in a counter run, whose copy calibration must be the
    # largest copy of the run (the LM head's weight is built by a 1 GB conversion kernel)
    kvc = tsel = lmh = asm = None
    if w.dtype == "bf16" and side:
        kvc = kv_compact_timing(st)
        log(f"kv_compact (after the step, not in it): {kvc['layers']} layers, {kvc['us']:.2f} us, "
            f"{kvc['algorithmic_bytes']} bytes moved")
    if side and not w.heads:
        asm = assemble_rows_timing(st)
        log(f"assemble_rows (before the step, not in it): {asm}")
    if side:
        tsel = tree_select_timing(w)
        log(f"tree_select (before the step, not in it): {tsel['pool']}, {tsel['us']:.2f} us")
        lmh = lm_head_stats_timing(w)
    if lmh:
        log(f"lm_head_stats (beside the step, not in it): {lmh['shape']}, {lmh['xperm_us']:.2f} us permute + "
            f"{lmh['us']:.2f} us + merge {lmh['merge_us']:.2f} us, {lmh['achieved_GBs']:.0f} GB/s; greedy verify "
            f"from the statistics {lmh['greedy_verify_us']:.2f} us, typical with its bonus draw "
            f"{lmh['typical_verify_us']:.2f} us; REJECT {lmh['reject_verify_us']}; WALK {lmh['walk_verify_us']}")
    res = {"w": w, "mode": mode, "a": a, "vi": vi, "hi": hi, "ti": ti, "ms_step": ms_step, "kernels": kernels,
           "kernels_frac": kernels_frac, "accept_len_mean": round(accept_mean, 3),
           "roofline": roof, "step_roofline": step_roof, "nsets": nsets, "use_graph": use_graph,
           "next_rows": {"kv_compact": kvc, "tree_select": tsel, "lm_head_stats": lmh, "assemble_rows": asm}}
    del st, sets, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the tree-verification step of one GPU's "
              "share); multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)
    import torch
    from tree_attention_verification_spec_amd import binding as sb

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sb.lib()
    side = not args.copy_calibration_mb or args.side_rows
    r = measure(args, args.config, args.steps, args.warmup, side)
    w, mode, ms_step = r["w"], r["mode"], r["ms_step"]

    # the other configuration the headline metric names (127 nodes at batch 16 beside the
    # 63-node batch-1 one), timed the same way, as an extra key of the same line
    also = {}
    for cfg in args.also:
        if cfg == args.config:
            continue
        ra = measure(args, cfg, max(20, args.steps // 4), min(args.warmup, 10), False, log_prefix="also: ")
        wa = ra["w"]
        also[wa.name] = {"value": round(wa.B * wa.N / (ra["ms_step"] * 1e-3), 1), "unit": "tree-nodes/s",
                         "ms_per_step": round(ra["ms_step"], 6), "rounds_per_s": round(1.0 / (ra["ms_step"] * 1e-3), 1),
                         "steps": max(20, args.steps // 4), "verify_mode": ra["mode"], "roofline": ra["roofline"],
                         "step_roofline": ra["step_roofline"], "accept_len_mean": ra["accept_len_mean"],
                         "kernels_us": {k: round(v * 1e3, 3) for k, v in ra["kernels"].items()},
                         "kernels_roofline_frac": ra["kernels_frac"]}
        del ra

    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb * (1 << 20)
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nb} bytes x 3")

    cpu = None
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        cpu = cpu_baseline(w, r["a"], r["vi"], r["hi"], r["ti"], mode, args.cpu_seconds / 2, threads)
        cpu["single_thread"] = cpu_baseline(w, r["a"], r["vi"], r["hi"], r["ti"], mode, args.cpu_seconds / 2, 1)
        log(f"cpu oracle: {cpu['value']} nodes/s on {threads} threads, {cpu['single_thread']['value']} on 1")

    nodes = w.B * w.N
    line = {
        "metric": METRIC,
        "value": round(nodes / (ms_step * 1e-3), 1),
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the pages' Llama-3-8B-class GQA, tree sizes, vocabularies)",
        "config": {"workload": w.name, "batch": w.B, "tree_nodes": w.N, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "prefix": list(w.prefix), "vocab": w.V, "verify_mode": mode,
                   "medusa_heads": w.heads, "rotating_copies": r["nsets"], "hip_graphs": r["use_graph"]},
        "rounds_per_s": round(1.0 / (ms_step * 1e-3), 1),
        "roofline": r["roofline"],
        "step_roofline": r["step_roofline"],
        "kernels_us": {k: round(v * 1e3, 3) for k, v in r["kernels"].items()},
        "kernels_roofline_frac": r["kernels_frac"],
        "accept_len_mean": r["accept_len_mean"],
        "also": also,
        "cpu_baseline": cpu,
        "next_rows": r["next_rows"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
