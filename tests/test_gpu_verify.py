"""GPU parity: spec_verify against the oracle.  accept_len, path, bonus token, per-node results and
error words are bit-exact; a sequence holding a decision within the stated margins of its
boundary (|u - min(1, T/D)| or |ln T - ln tau| below 1e-4, or a bonus draw within 1e-9
(relative) of a CDF step) is counted separately."""

import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import compare_verify, dev, host, need_gpu

pytestmark = pytest.mark.gpu

MODE = {"greedy": oracle.MODE_GREEDY, "typical": oracle.MODE_TYPICAL, "reject": oracle.MODE_REJECT}


def _run(w, mode, vi, parents, n_nodes, eps=0.09, delta=0.3, max_depth=None):
    need_gpu()
    eps32, delta32 = float(np.float32(eps)), float(np.float32(delta))
    if max_depth is None:
        max_depth = w.N - 1
    use_draft = mode == "reject"
    got = sb.spec_verify(dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents.astype(np.int32)),
                         dev(vi["uniforms"]), mode,
                         draft_probs=dev(vi["draft_probs"]) if use_draft else None,
                         draft_row=dev(vi["draft_row"]) if use_draft else None,
                         t2d=dev(vi["t2d"]) if (use_draft and vi["t2d"] is not None) else None,
                         n_nodes=dev(n_nodes.astype(np.int32)), eps=eps32, delta=delta32, max_depth=max_depth)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    ref = oracle.verify(vi["target_logits"], vi["tokens"], parents, vi["uniforms"], MODE[mode],
                        draft_probs=vi["draft_probs"], draft_row=vi["draft_row"], t2d=vi["t2d"],
                        n_nodes=n_nodes, eps=eps32, delta=delta32, max_depth=max_depth)
    return got, ref


def _case(w):
    parents, n_nodes = wl.trees(w)
    return parents, n_nodes, wl.verify_inputs(w, parents)


@pytest.mark.parametrize("cfg,mode", [(1, "greedy"), (1, "reject"), (2, "typical"), (2, "reject"), (3, "reject"),
                                      (4, "reject")])
def test_configs(cfg, mode):
    w = wl.config(cfg)
    parents, n_nodes, vi = _case(w)
    got, ref = _run(w, mode, vi, parents, n_nodes)
    ex = compare_verify(got, ref, n_nodes)
    print(f"cfg{cfg} {mode}: mean accept_len {ref['accept_len'].mean():.2f}, excused {ex}/{w.B}")


SMALL = [
    dict(B=16, N=37, V=5000),
    dict(B=8, N=63, V=2049, sigma_logits=1.0),
    dict(B=6, N=127, V=300, n_nodes_range=(1, 127), sigma_logits=0.5),
    dict(B=4, N=256, V=4099, tree=("random", 8)),
    dict(B=5, N=30, V=800, Vd=333),
    dict(B=9, N=10, V=1, tree=("random", 3)),
    dict(B=7, N=12, V=70000, draft_rows="per_depth", tree=("bfs", (3, 2, 2))),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("mode", ["greedy", "typical", "reject"])
def test_small(case, mode):
    w = wl.custom(seed=3000 + case, **SMALL[case])
    parents, n_nodes, vi = _case(w)
    for eps, delta in ((0.09, 0.3), (0.01, float("inf")), (2.0, float("inf"))):
        got, ref = _run(w, mode, vi, parents, n_nodes, eps=eps, delta=delta)
        compare_verify(got, ref, n_nodes)
        if mode != "typical":
            break


@pytest.mark.parametrize("chunk", ["4096", "16384"])
@pytest.mark.parametrize("case", [0, 2, 6])
def test_row_chunk_sizes(tune, chunk, case):
    """The row pass at each chunk size its tuning override allows (8192 is the default)."""
    tune(verify_chunk=int(chunk))
    w = wl.custom(seed=3000 + case, **SMALL[case])
    parents, n_nodes, vi = _case(w)
    for mode in ("greedy", "typical", "reject"):
        got, ref = _run(w, mode, vi, parents, n_nodes)
        compare_verify(got, ref, n_nodes)


@pytest.mark.parametrize("listed", ["0", "1"])
@pytest.mark.parametrize("case", [0, 2, 3, 4, 6])
def test_row_pass_listed_or_per_chunk(tune, listed, case):
    """The row pass as one workgroup per (sequence, node, chunk), or as a listing of the rows
    with children followed by one workgroup per listed (row, chunk) item (large problems by
    default): both, forced, on every mode."""
    tune(verify_rows_list=int(listed))
    w = wl.custom(seed=3000 + case, **SMALL[case])
    parents, n_nodes, vi = _case(w)
    for mode in ("greedy", "typical", "reject"):
        got, ref = _run(w, mode, vi, parents, n_nodes)
        compare_verify(got, ref, n_nodes)


@pytest.mark.parametrize("store", ["0", "1"])
@pytest.mark.parametrize("case", [0, 1, 3, 6])
def test_draw_weights_stored_or_recomputed(tune, store, case):
    """The one-wave bonus draw either scans per-token weights stored by the bonus pass (forced)
    or picks a 64-token group from the group sums and recomputes one weight per lane (the
    default): both paths on every mode."""
    tune(verify_store_w=int(store))
    w = wl.custom(seed=3000 + case, **SMALL[case])
    parents, n_nodes, vi = _case(w)
    for mode in ("greedy", "typical", "reject"):
        got, ref = _run(w, mode, vi, parents, n_nodes)
        compare_verify(got, ref, n_nodes)


@pytest.mark.parametrize("store", ["0", "1"])
def test_wide_vocabulary_workgroup_draw(tune, store):
    """A vocabulary of 300000 tokens is more than 64 bonus chunks of 4096, so the draw runs on a
    workgroup with block scans (stored weights or recomputed ones) instead of one wave."""
    tune(verify_store_w=int(store))
    w = wl.custom(seed=3050, B=2, N=20, V=300_000, sigma_logits=0.5, tree=("random", 4))
    parents, n_nodes, vi = _case(w)
    for mode in ("typical", "reject"):
        got, ref = _run(w, mode, vi, parents, n_nodes)
        compare_verify(got, ref, n_nodes)


@pytest.mark.parametrize("store", ["0", "1"])
@pytest.mark.parametrize("V", [9000, 300_000])
def test_zero_residual_draws_from_target(tune, store, V):
    """Draft probabilities of 2 everywhere: each node test accepts with T/D <= 1/2 and every
    residual relu(T - D) is zero, so a rejection's bonus token is drawn from T at the kept node
    (the zero-mass reading), on every draw kernel: one wave over stored weights or over group
    sums (9000 tokens), a workgroup over stored or recomputed weights (300000 tokens)."""
    tune(verify_store_w=int(store))
    w = wl.custom(seed=3100, B=6 if V < 100_000 else 3, N=40, V=V, tree=("random", 5))
    parents, n_nodes, vi = _case(w)
    vi = dict(vi)
    vi["draft_probs"] = np.full_like(vi["draft_probs"], 2.0)
    got, ref = _run(w, "reject", vi, parents, n_nodes)
    assert (ref["accept_len"] < 5).sum() >= 3          # rejections happened
    compare_verify(got, ref, n_nodes)


@pytest.mark.parametrize("listed", ["0", "1"])
def test_max_depth_and_errors(tune, listed):
    need_gpu()
    tune(verify_rows_list=int(listed))
    w = wl.custom(seed=41, B=8, N=20, V=64, tree=("random", 6))
    parents, n_nodes, vi = _case(w)
    vi = dict(vi)
    tokens = vi["tokens"].copy()
    tokens[1, 5] = 64                                   # token out of range
    tokens[2, 3] = -2
    vi["tokens"] = tokens
    dr = vi["draft_row"].copy()
    dr[3, 7] = vi["R"]                                  # draft row out of range
    vi["draft_row"] = dr
    logits = vi["target_logits"].copy()
    logits[4, 0, 9] = np.nan                            # root row is always read
    vi["target_logits"] = logits
    parents = parents.copy()
    parents[5, 4] = 9                                   # parent after child
    parents[6, 0] = 3                                   # bad root
    n_nodes = n_nodes.copy()
    n_nodes[7] = 21                                     # too many nodes
    for mode in ("greedy", "typical", "reject"):
        for md in (w.N - 1, 2):
            got, ref = _run(w, mode, vi, parents, n_nodes, max_depth=md)
            assert (ref["err"] != 0).sum() >= 5
            compare_verify(got, ref, n_nodes)


def test_chi_square_gpu():
    """The GPU path draws the same distribution tests as the oracle: a 2-node chain with x ~ D
    emits its first token with the law of T_root (chi-square, 1e5 seeded trials)."""
    need_gpu()
    from scipy import stats as sps
    from scipy.special import softmax
    V, trials = 8, 100_000
    g = wl.rng(0, wl.S_TRIALS, 4242)
    logits = (g.standard_normal((3, V)) * 1.5).astype(np.float32)
    T = softmax(logits.astype(np.float64), axis=-1)
    D = softmax(g.standard_normal((2, V)) * 1.5, axis=-1).astype(np.float32)
    x1 = g.choice(V, size=trials, p=D[0] / D[0].sum(dtype=np.float64))
    x2 = g.choice(V, size=trials, p=D[1] / D[1].sum(dtype=np.float64))
    u = g.random((trials, 3), dtype=np.float32)
    tokens = np.stack([np.full(trials, -1), x1, x2], 1).astype(np.int32)
    parents = np.tile(np.array([-1, 0, 1], np.int32), (trials, 1))
    got = sb.spec_verify(dev(np.ascontiguousarray(np.broadcast_to(logits, (trials, 3, V)))), dev(tokens),
                         dev(parents), dev(u), "reject",
                         draft_probs=dev(np.ascontiguousarray(np.broadcast_to(D, (trials, 2, V)))),
                         draft_row=dev(np.tile(np.array([-1, 0, 1], np.int32), (trials, 1))))
    acc = host(got["accept_len"])
    bonus = host(got["bonus"])
    first = np.where(acc >= 1, x1, bonus)
    assert sps.chisquare(np.bincount(first, minlength=V), T[0] * trials).pvalue > 1e-3
    # and the GPU agrees with the oracle on a slice of the same trials
    sl = slice(0, 3000)
    ref = oracle.verify(np.broadcast_to(logits, (3000, 3, V)), tokens[sl], parents[sl], u[sl], oracle.MODE_REJECT,
                        draft_probs=np.broadcast_to(D, (3000, 2, V)), draft_row=np.tile([-1, 0, 1], (3000, 1)))
    gsl = {k: host(v)[sl] for k, v in got.items()}
    compare_verify(gsl, ref, np.full(3000, 3))
