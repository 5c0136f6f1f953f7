"""GPU parity of spec_lm_head_stats (the target LM head fused with the verify row statistics)
against oracle.lm_head_stats.

Tolerance, derived from the arithmetic: bf16 x bf16 products are exact in fp32 and the GPU sums
Dm of them in fp32 in some order, so every logit is within
    delta_p = (Dm + 2) * 2^-24 * max_v sum_k |h_p[k]| |W[v, k]|
of the exact one (the standard bound for a sum of Dm terms in any order, with slack).  Then
row_max and cand_logit are within delta_p; the lowest argmax is exact unless the oracle's two
best logits are within 2 delta_p (then the GPU's choice must hold a logit within 2 delta_p of
the max); S = sum exp(l - max) is within a factor exp(+-2 delta_p) (+ fp32 exp rounding); the
entropy ln S - A / S within 4 delta_p (H + 1).  Error words and NaN patterns are exact."""

import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu


def bound(h, W):
    """delta per (b, i): (Dm + 2) 2^-24 max_v sum_k |h||W| (fp32 product, inflated by 1 %)."""
    B, N, Dm = h.shape
    absW = torch.from_numpy(np.abs(W)).float()
    s = torch.from_numpy(np.abs(h).reshape(B * N, Dm)).float() @ absW.T
    return ((Dm + 2) * 2.0 ** -24 * 1.01 * s.max(dim=1).values.double().numpy()).reshape(B, N)


def run_both(inp, n_nodes=None, what=""):
    need_gpu()
    h, W, par, tok = inp["hidden"], inp["W"], inp["parents"], inp["tokens"]
    B, N, Dm = h.shape
    print(f"lm_head_stats {what}: B={B} N={N} Dm={Dm} V={W.shape[0]}", flush=True)
    got = sb.spec_lm_head_stats(dev(h, torch.bfloat16), dev(W, torch.bfloat16), dev(par), dev(tok),
                                n_nodes=None if n_nodes is None else dev(n_nodes))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    ref = oracle.lm_head_stats(h, W, par, tok, n_nodes=n_nodes)
    assert np.array_equal(got["err"], ref["err"]), f"{what}: err {got['err']} vs {ref['err']}"
    ok = np.isfinite(ref["row_max"])
    for key in ("row_max", "row_sum", "row_ent", "cand_logit"):
        assert np.array_equal(np.isnan(got[key]), np.isnan(ref[key])), f"{what}: {key} NaN pattern"
    assert np.array_equal(got["row_argmax"][~ok], ref["row_argmax"][~ok])
    d = bound(h, W)
    worst = {}
    for b, i in zip(*np.nonzero(ok)):
        dl = d[b, i]
        row = ref["logits"][b, i]
        m = ref["row_max"][b, i]
        e_max = abs(got["row_max"][b, i] - m)
        assert e_max <= dl, f"{what}: row_max ({b},{i}) off by {e_max:.3e} > {dl:.3e}"
        ga, ra = int(got["row_argmax"][b, i]), int(ref["row_argmax"][b, i])
        if ga != ra:
            second = np.partition(row, -2)[-2]
            assert m - second <= 2 * dl and row[ga] >= m - 2 * dl, f"{what}: argmax ({b},{i}) {ga} vs {ra}"
        S, A = ref["row_sum"][b, i], ref["row_ent"][b, i]
        gS, gA = got["row_sum"][b, i], got["row_ent"][b, i]
        assert abs(gS - S) <= (np.expm1(2 * dl) + 1e-6) * S, f"{what}: row_sum ({b},{i}) {gS} vs {S}"
        H, gH = np.log(S) - A / S, np.log(gS) - gA / gS
        assert abs(gH - H) <= 4 * dl * (H + 1) + 1e-6, f"{what}: entropy ({b},{i}) {gH} vs {H}"
        if i > 0:
            e_c = abs(got["cand_logit"][b, i] - ref["cand_logit"][b, i])
            assert e_c <= dl, f"{what}: cand_logit ({b},{i}) off by {e_c:.3e} > {dl:.3e}"
            worst["cand"] = max(worst.get("cand", 0.0), e_c)
        worst["max"] = max(worst.get("max", 0.0), e_max)
        worst["bound"] = max(worst.get("bound", 0.0), dl)
    print(f"  worst |d max| {worst.get('max', 0):.2e}, |d cand| {worst.get('cand', 0):.2e}, "
          f"bound {worst.get('bound', 0):.2e}", flush=True)
    return got, ref


@pytest.mark.parametrize("B,N,Dm,V", [(1, 1, 128, 1), (1, 5, 128, 37), (1, 16, 128, 64), (1, 17, 256, 65),
                                      (2, 16, 256, 1000), (3, 11, 128, 5000), (4, 16, 384, 2048),
                                      (1, 64, 512, 4099), (1, 65, 128, 700), (2, 256, 256, 1500),
                                      (8, 127, 512, 4099), (16, 127, 256, 3000), (3, 43, 128, 1000),
                                      (16, 256, 128, 700)])
def test_small(B, N, Dm, V):
    inp = wl.lm_head_inputs(seed=40 + B + N + V, B=B, N=N, Dm=Dm, V=V)
    run_both(inp, what=f"small {B}x{N} Dm{Dm} V{V}")


def test_ragged_and_errors():
    inp = wl.lm_head_inputs(seed=9, B=4, N=12, Dm=256, V=3000)
    inp["parents"][1, 0] = 0
    inp["parents"][2, 5] = 9
    inp["tokens"][3, 4] = 3000
    run_both(inp, n_nodes=np.array([7, 12, 12, 12], dtype=np.int32), what="errors")
    inp = wl.lm_head_inputs(seed=10, B=4, N=12, Dm=256, V=3000)
    run_both(inp, n_nodes=np.array([12, 0, 1, 13], dtype=np.int32), what="ragged")


def test_ties():
    """Columns of W that repeat the best logit: the lowest id wins, on the GPU as in the oracle."""
    inp = wl.lm_head_inputs(seed=12, B=1, N=8, Dm=128, V=700)
    W = inp["W"]
    W[[13, 200, 511, 699]] = W[600]
    inp["hidden"][0, :] = np.sign(W[600])[None, :] * np.abs(inp["hidden"][0, :])   # make row 600 win
    got, ref = run_both(inp, what="ties")
    assert (ref["row_argmax"][0] == 13).all()
    assert np.isin(got["row_argmax"][0], [13, 200, 511, 600, 699]).all()
    print(f"  GPU argmax on the tied rows: {got['row_argmax'][0].tolist()}", flush=True)


def test_llama3_8b_shape():
    """The 63-node batch-1 workload's shapes: hidden 4096, vocabulary 128256 (a 1 GB LM head)."""
    inp = wl.lm_head_inputs(seed=2, B=1, N=63, Dm=4096, V=128256)
    run_both(inp, what="llama3-8b B1 N63")


@pytest.mark.parametrize("seed,B,N,Dm,V", [(21, 1, 63, 4096, 128256), (22, 4, 16, 512, 3000), (23, 2, 30, 256, 777),
                                            (24, 16, 127, 256, 2000)])
def test_greedy_round_from_statistics(seed, B, N, Dm, V):
    """LM head statistics then greedy verification, both on the GPU, against the oracle's logits
    through oracle.verify (GREEDY).  Candidate tokens are the oracle's argmax of the parent's row
    for about 70 % of the nodes, so paths are long.  Greedy outcomes depend on the row arg-maxima
    only: a sequence whose GPU arg-maxima all equal the oracle's must match exactly; one where
    an arg-maximum differs (allowed only within the fp32 accumulation bound, checked here) is
    counted, not compared."""
    need_gpu()
    inp = wl.lm_head_inputs(seed=seed, B=B, N=N, Dm=Dm, V=V, max_depth=6)
    ref_stats = oracle.lm_head_stats(inp["hidden"], inp["W"], inp["parents"], inp["tokens"])
    g = np.random.default_rng(seed)
    tok = inp["tokens"].copy()
    for b in range(B):
        for c in range(1, N):
            if g.random() < 0.7:
                tok[b, c] = ref_stats["row_argmax"][b, inp["parents"][b, c]]
    inp["tokens"] = tok
    n_nodes = np.array([N - (b % 3) for b in range(B)], dtype=np.int32)
    print(f"greedy round B={B} N={N} Dm={Dm} V={V}", flush=True)
    st = sb.spec_lm_head_stats(dev(inp["hidden"], torch.bfloat16), dev(inp["W"], torch.bfloat16),
                               dev(inp["parents"]), dev(tok), n_nodes=dev(n_nodes))
    ver = sb.spec_verify_greedy_stats(st["row_argmax"], dev(tok), dev(inp["parents"]), V, n_nodes=dev(n_nodes))
    torch.cuda.synchronize()
    ref = oracle.lm_head_stats(inp["hidden"], inp["W"], inp["parents"], tok, n_nodes=n_nodes)
    logits = np.nan_to_num(ref["logits"], nan=0.0)
    rv = oracle.verify(logits, tok, inp["parents"], np.zeros((B, N), np.float32), oracle.MODE_GREEDY,
                       n_nodes=n_nodes)
    d = bound(inp["hidden"], inp["W"])
    got = {k: host(v) for k, v in ver.items()}
    gam = host(st["row_argmax"])
    compared = 0
    for b in range(B):
        nb = int(n_nodes[b])
        differ = np.flatnonzero(gam[b, :nb] != ref["row_argmax"][b, :nb])
        for i in differ:                    # a different argmax only within the accumulation bound
            row = ref["logits"][b, i]
            assert row[gam[b, i]] >= row.max() - 2 * d[b, i], f"sequence {b} row {i}: argmax off"
        if differ.size:
            continue
        compared += 1
        assert int(got["err"][b]) == int(rv["err"][b])
        assert int(got["accept_len"][b]) == int(rv["accept_len"][b]), f"sequence {b}: accept_len"
        assert np.array_equal(got["path"][b], rv["path"][b]), f"sequence {b}: path"
        assert int(got["bonus"][b]) == int(rv["bonus"][b]), f"sequence {b}: bonus"
        assert np.array_equal(got["node_accept"][b], rv["node_accept"][b]), f"sequence {b}: node_accept"
    print(f"  compared {compared} of {B} sequences; accept_len {got['accept_len'].tolist()}", flush=True)
    assert compared >= 1


def test_greedy_stats_errors():
    """Error words and the empty sequence, from arg-maxima given directly."""
    need_gpu()
    B, N, V = 6, 8, 50
    par = np.tile(np.array([-1, 0, 0, 1, 1, 2, 3, 6], np.int32), (B, 1))
    tok = np.tile(np.array([-1, 5, 7, 9, 5, 1, 2, 3], np.int32), (B, 1))
    am = np.tile(np.array([5, 9, 1, 2, 0, 0, 3, 4], np.int32), (B, 1))
    par[1, 0] = 3
    par[2] = np.arange(-1, 7, dtype=np.int32)          # a chain: node 5 is deeper than max_depth
    par[2, 4] = 4
    tok[3, 5] = 50
    n_nodes = np.array([8, 8, 8, 8, 0, 9], np.int32)
    got = sb.spec_verify_greedy_stats(dev(am), dev(tok), dev(par), V, n_nodes=dev(n_nodes), max_depth=4)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    # the oracle on logits whose argmax is am (one-hot rows)
    logits = np.zeros((B, N, V))
    for b in range(B):
        for i in range(N):
            logits[b, i, am[b, i]] = 1.0
    rv = oracle.verify(logits, tok, par, np.zeros((B, N), np.float32), oracle.MODE_GREEDY, n_nodes=n_nodes,
                       max_depth=4)
    for key in ("err", "accept_len", "bonus"):
        assert np.array_equal(got[key], rv[key]), f"{key}: {got[key]} vs {rv[key]}"
    assert np.array_equal(got["path"], rv["path"]) and np.array_equal(got["node_accept"], rv["node_accept"])
    assert [oracle.decode_err(e) for e in rv["err"]] == [(0, 0), (0, oracle.ERR_ROOT), (4, oracle.ERR_PARENT),
                                                         (5, oracle.ERR_TOKEN), (0, 0), (0, oracle.ERR_NNODES)]
    assert int(rv["accept_len"][0]) == 4 and int(rv["bonus"][0]) == 4   # path 0 -> 1 -> 3 -> 6 -> 7


def measured_error(st, ref, b, nb):
    """The error of this run's statistics in sequence b, against the oracle's exact values:
    (largest |d max|, |d cand_logit|, |d ln S|, |d entropy|) over its rows.  Each is asserted
    within the worst-case bound elsewhere; the decisions are excused only within these."""
    ok = np.arange(nb)
    e_max = float(np.abs(st["row_max"][b, ok] - ref["row_max"][b, ok]).max())
    e_cand = float(np.abs(st["cand_logit"][b, 1:nb] - ref["cand_logit"][b, 1:nb]).max()) if nb > 1 else 0.0
    e_lnS = float(np.abs(np.log(st["row_sum"][b, ok]) - np.log(ref["row_sum"][b, ok])).max())
    H = np.log(ref["row_sum"][b, ok]) - ref["row_ent"][b, ok] / ref["row_sum"][b, ok]
    gH = np.log(st["row_sum"][b, ok]) - st["row_ent"][b, ok] / st["row_sum"][b, ok]
    e_H = float(np.abs(gH - H).max())
    return e_max, e_cand, e_lnS, e_H


# fp32 rounding of the GPU's own exp(l - max) / S and of the threshold (relative)
ROUND = 4e-7
# per-logit error of a whole row, estimated from the sampled logits (the row maxima and the
# candidates' logits) with a safety factor: the walk and the bonus draws read every logit
ROW_SAFETY = 8.0


@pytest.mark.parametrize("mode", ["greedy", "typical", "reject", "reject_row", "walk", "reject_t2d", "walk_t2d"])
@pytest.mark.parametrize("seed,B,N,Dm,V,hscale", [(41, 2, 40, 256, 3000, 8.0), (42, 4, 16, 128, 700, 12.0),
                                                   (43, 1, 63, 4096, 128256, 1.0), (45, 4, 63, 4096, 128256, 1.0),
                                                   (44, 8, 127, 256, 2000, 8.0)])
def test_verify_from_hidden_states(mode, seed, B, N, Dm, V, hscale):
    """spec_verify_lm_head against oracle.verify on the oracle's exact logits.

    Decisions are excused only within the error this run actually makes: the GPU's statistics
    (row max, candidate logits, S, entropy; the same kernels spec_verify_lm_head runs) are read
    through spec_lm_head_stats and compared with the oracle's, each asserted within the
    worst-case fp32 bound, and the measured differences set the bands.  With d = |d cand| +
    |d max| + |d ln S| (the error of ln T_p[x]): REJECT excuses |u - min(1, T/D)| < 2 d + 4e-7;
    TYPICAL |ln T - ln tau| < 2 (d + |d H|) + 4e-7; GREEDY compares sequences whose row
    arg-maxima all equal the oracle's.  Reading a whole row (WALK, the bonus draws), the
    per-logit error is taken as 8 x the largest sampled one (e): WALK excuses sibling tests
    within 12 e + 1e-6 (relative); the TYPICAL and leaf bonus must lie in the oracle's CDF step
    widened by 4 (e + |d ln S|), a residual bonus by that over the residual's mass; WALK's bonus
    must equal the oracle's where its CDF margin exceeds 100 e.  Every mode must compare at
    least one sequence, at every shape.  reject_row drafts random tokens with draft rows peaked
    on them and node uniforms in [0.1, 1), so the root's children are rejected and the bonus is
    a residual draw over the stored row.  *_t2d: the draft rows live on a smaller vocabulary,
    reached through a random map t2d in which about a third of the target tokens have no draft
    id (-1: no draft mass).  [GUIDE] "棄却サンプリング：出力品質を保証する"."""
    need_gpu()
    inp = wl.lm_head_inputs(seed=seed, B=B, N=N, Dm=Dm, V=V, max_depth=6)
    inp["hidden"] = wl.round_bf16(inp["hidden"] * np.float32(hscale))
    ref0 = oracle.lm_head_stats(inp["hidden"], inp["W"], inp["parents"], inp["tokens"])
    g = np.random.default_rng(seed)
    tok = inp["tokens"].copy()
    for b in range(B):
        for c in range(1, N):
            if g.random() < 0.6 and mode != "reject_row":
                tok[b, c] = ref0["row_argmax"][b, inp["parents"][b, c]]
    unif = g.random((B, N), dtype=np.float32)
    n_nodes = np.array([N - (b % 2) for b in range(B)], dtype=np.int32)
    eps, delta = float(np.float32(0.09)), float(np.float32(0.3))
    draft = drow = t2d = None
    if mode.startswith(("reject", "walk")):
        # per-parent draft rows: D_p = softmax(l_p + N(0, 0.5)) of the oracle's logits (inputs only)
        x = np.nan_to_num(ref0["logits"], nan=0.0) + g.standard_normal(ref0["logits"].shape) * 0.5
        e = np.exp(x - x.max(axis=2, keepdims=True))
        draft = e / e.sum(axis=2, keepdims=True)
        del x, e
        drow = np.maximum(inp["parents"], 0).astype(np.int32)
        if mode == "reject_row":
            unif[:, 1:] = np.float32(0.1) + np.float32(0.9) * unif[:, 1:]   # clear of T/D ~ 0
            for b in range(B):
                for c in range(1, N):
                    draft[b, drow[b, c], tok[b, c]] += 1.0
            draft /= draft.sum(axis=2, keepdims=True)
        draft = draft.astype(np.float32)
        draft_t = draft                                  # the draft rows on the target vocabulary
        if mode.endswith("_t2d"):
            Vd = 2 * V // 3 + 1
            perm = g.permutation(V)
            t2d = np.where(perm < Vd, perm, -1).astype(np.int32)
            dd = np.zeros((B, N, Vd), np.float64)
            on = t2d >= 0
            dd[:, :, t2d[on]] = draft[:, :, on]
            dd /= dd.sum(axis=2, keepdims=True)
            draft = dd.astype(np.float32)
            draft_t = np.where(on[None, None, :], draft[:, :, np.maximum(t2d, 0)], 0.0).astype(np.float32)
    del ref0
    print(f"verify_lm_head {mode} B={B} N={N} Dm={Dm} V={V}", flush=True)
    got = sb.spec_verify_lm_head(dev(inp["hidden"], torch.bfloat16), dev(inp["W"], torch.bfloat16), dev(tok),
                                 dev(inp["parents"]), dev(unif), mode.split("_")[0], n_nodes=dev(n_nodes),
                                 eps=eps, delta=delta,
                                 draft_probs=None if draft is None else dev(draft),
                                 draft_row=None if drow is None else dev(drow),
                                 t2d=None if t2d is None else dev(t2d))
    # the statistics the decisions were made from (same kernels, same inputs)
    st = sb.spec_lm_head_stats(dev(inp["hidden"], torch.bfloat16), dev(inp["W"], torch.bfloat16), dev(inp["parents"]),
                               dev(tok), n_nodes=dev(n_nodes))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    st = {k: host(v) for k, v in st.items()}
    ref = oracle.lm_head_stats(inp["hidden"], inp["W"], inp["parents"], tok, n_nodes=n_nodes)
    logits = np.nan_to_num(ref["logits"], nan=0.0)
    m_id = {"greedy": oracle.MODE_GREEDY, "typical": oracle.MODE_TYPICAL, "reject": oracle.MODE_REJECT,
            "walk": oracle.MODE_WALK}[mode.split("_")[0]]
    rv = oracle.verify(logits, tok, inp["parents"], unif, m_id, n_nodes=n_nodes, eps=eps, delta=delta,
                       draft_probs=draft, draft_row=drow, t2d=t2d)
    d = bound(inp["hidden"], inp["W"])
    gam = st["row_argmax"]
    compared = bonus_checked = resid_checked = 0
    for b in range(B):
        nb = int(n_nodes[b])
        assert int(got["err"][b]) == int(rv["err"][b])
        e_max, e_cand, e_lnS, e_H = measured_error(st, ref, b, nb)
        dseq = float(d[b, :nb].max())
        assert e_max <= dseq and e_cand <= dseq, f"sequence {b}: statistics outside the fp32 bound"
        d_lnT = e_cand + e_max + e_lnS
        e_row = ROW_SAFETY * max(e_max, e_cand, 1e-9)
        if mode == "greedy":
            differ = np.flatnonzero(gam[b, :nb] != ref["row_argmax"][b, :nb])
            for i in differ:
                row = ref["logits"][b, i]
                assert row[gam[b, i]] >= row.max() - 2 * d[b, i], f"sequence {b} row {i}: argmax off"
            if differ.size:
                continue
        elif mode == "typical":
            if np.any(rv["margin"][b, 1:nb] < 2 * (d_lnT + e_H) + ROUND):
                continue
        elif mode.startswith("walk"):
            if np.any(rv["margin"][b, 1:nb] < 12 * e_row + 1e-6):
                continue
        elif np.any(rv["margin"][b, 1:nb] < 2 * d_lnT + ROUND):
            continue
        compared += 1
        assert np.array_equal(got["node_accept"][b], rv["node_accept"][b]), f"sequence {b}: node_accept"
        assert int(got["accept_len"][b]) == int(rv["accept_len"][b]), f"sequence {b}: accept_len"
        assert np.array_equal(got["path"][b], rv["path"][b]), f"sequence {b}: path"
        if mode == "greedy":
            assert int(got["bonus"][b]) == int(rv["bonus"][b]), f"sequence {b}: bonus"
            bonus_checked += 1
        elif mode.startswith("walk"):
            if rv["bonus_margin"][b] > 100 * e_row:
                assert int(got["bonus"][b]) == int(rv["bonus"][b]), f"sequence {b}: walk bonus"
                bonus_checked += 1
            elif int(got["bonus"][b]) != int(rv["bonus"][b]):
                print(f"  sequence {b}: walk bonus {int(got['bonus'][b])} vs oracle {int(rv['bonus'][b])} "
                      f"(CDF margin {rv['bonus_margin'][b]:.1e})")
        else:
            m = int(rv["m"][b])
            row = logits[b, m]
            T = np.exp(row - row.max())
            T = T / T.sum()
            q, tol = T, 4 * (e_row + e_lnS) + 1e-12
            kids = [c for c in range(1, nb) if inp["parents"][b, c] == m]
            if mode.startswith("reject") and kids:
                res = np.maximum(T - draft_t[b, drow[b, kids[0]]].astype(np.float64), 0.0)
                if res.sum() > 0:
                    q, tol = res, 4 * (e_row + e_lnS) / res.sum() + 1e-12
                    resid_checked += 1
            C = np.cumsum(q) / q.sum()
            t = int(got["bonus"][b])
            assert 0 <= t < V
            lo = C[t - 1] if t > 0 else 0.0
            assert lo <= unif[b, 0] + tol and C[t] >= unif[b, 0] - tol, \
                f"sequence {b}: bonus {t} outside the oracle's CDF step (u {unif[b, 0]}, [{lo}, {C[t]}], tol {tol:.1e})"
            bonus_checked += 1
            if int(rv["bonus"][b]) != t:
                print(f"  sequence {b}: bonus {t} vs oracle {int(rv['bonus'][b])} (u within {tol:.1e} of a step)")
    print(f"  compared {compared} of {B} sequences, {bonus_checked} bonus tokens; accept_len "
          f"{got['accept_len'].tolist()}; oracle {rv['accept_len'].tolist()}", flush=True)
    assert compared >= 1, f"{mode}: no sequence compared"
    if mode == "reject_row":
        print(f"  residual draws checked: {resid_checked}", flush=True)
        assert resid_checked >= 1


@pytest.mark.parametrize("mode", ["reject", "walk"])
def test_verify_from_hidden_states_draft_errors(mode):
    """Error words of REJECT and WALK from hidden states equal the oracle's: a draft row out of
    range, a t2d entry outside [-1, Vd), and (WALK only) siblings drafted from different rows.
    Sequences without an error must still match wherever no decision is within the bound."""
    need_gpu()
    B, N, Dm, V, Vd = 5, 12, 128, 500, 400
    inp = wl.lm_head_inputs(seed=77, B=B, N=N, Dm=Dm, V=V, max_depth=4)
    g = np.random.default_rng(77)
    tok = inp["tokens"].copy()
    par = inp["parents"]
    tok[:, 1:] = g.integers(0, V - 1, size=(B, N - 1))          # token V - 1 is kept for sequence 2
    t2d = np.where(np.arange(V) < Vd, np.arange(V), -1).astype(np.int32)
    t2d[V - 1] = Vd + 3                                           # a map entry out of range
    tok[2, 5] = V - 1
    draft = g.random((B, N, Vd)).astype(np.float32)
    draft /= draft.sum(axis=2, keepdims=True)
    drow = np.maximum(par, 0).astype(np.int32)
    drow[1, 3] = N                                                # a draft row out of range
    kids0 = [c for c in range(1, N) if par[3, c] == 0]
    if len(kids0) > 1:
        drow[3, kids0[1]] = (drow[3, kids0[0]] + 1) % N          # siblings from different rows
    unif = g.random((B, N), dtype=np.float32)
    print(f"verify_lm_head {mode} draft errors", flush=True)
    got = sb.spec_verify_lm_head(dev(inp["hidden"], torch.bfloat16), dev(inp["W"], torch.bfloat16), dev(tok),
                                 dev(par), dev(unif), mode, draft_probs=dev(draft), draft_row=dev(drow),
                                 t2d=dev(t2d))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    ref = oracle.lm_head_stats(inp["hidden"], inp["W"], par, tok)
    logits = np.nan_to_num(ref["logits"], nan=0.0)
    m_id = oracle.MODE_REJECT if mode == "reject" else oracle.MODE_WALK
    rv = oracle.verify(logits, tok, par, unif, m_id, draft_probs=draft, draft_row=drow, t2d=t2d)
    assert np.array_equal(got["err"], rv["err"]), f"err {got['err']} vs {rv['err']}"
    codes = [oracle.decode_err(int(e)) for e in rv["err"]]
    assert codes[1] == (3, oracle.ERR_DRAFTROW) and codes[2] == (5, oracle.ERR_MAP)
    if mode == "walk" and len(kids0) > 1:
        assert codes[3][1] == oracle.ERR_DRAFTROW
    d = bound(inp["hidden"], inp["W"])
    for b in range(B):
        if rv["err"][b] != 0:
            continue
        if np.any(rv["margin"][b, 1:] < 6 * float(d[b].max()) + 1e-9):
            continue
        assert int(got["accept_len"][b]) == int(rv["accept_len"][b]), f"sequence {b}: accept_len"
        assert np.array_equal(got["path"][b], rv["path"][b]), f"sequence {b}: path"
    print(f"  err words {[hex(int(e)) for e in got['err']]}", flush=True)
