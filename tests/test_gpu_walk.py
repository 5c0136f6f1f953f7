"""GPU parity of spec_verify's WALK mode (the tree-lossless sibling-residual walk) against the
oracle: accept_len, path, bonus, node_accept (the path) and error words bit-exact per sequence,
sequences holding a decision near its boundary counted separately.  Node tests are excused below
a relative distance of 1e-4 (the oracle's walk margin); residual bonus draws below 1e-7 of the
CDF total, since the residual's scale comes from fp32-exp sums (relative error near 1e-9, times
1/f for a residual of mass f); draws from T keep the fp64 bound of the other modes."""

import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import compare_verify, dev, host, need_gpu

pytestmark = pytest.mark.gpu

WALK_BONUS_MARGIN = 1e-7


def _run(vi, parents, n_nodes, max_depth):
    need_gpu()
    got = sb.spec_verify(dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents.astype(np.int32)),
                         dev(vi["uniforms"]), "walk", draft_probs=dev(vi["draft_probs"]),
                         draft_row=dev(vi["draft_row"]),
                         t2d=dev(vi["t2d"]) if vi["t2d"] is not None else None,
                         n_nodes=dev(n_nodes.astype(np.int32)), max_depth=max_depth)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    ref = oracle.verify(vi["target_logits"], vi["tokens"], parents, vi["uniforms"], oracle.MODE_WALK,
                        draft_probs=vi["draft_probs"], draft_row=vi["draft_row"], t2d=vi["t2d"],
                        n_nodes=n_nodes, max_depth=max_depth)
    return got, ref


def _check(w, max_depth=None):
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    md = w.N - 1 if max_depth is None else max_depth
    got, ref = _run(vi, parents, n_nodes, md)
    ex = compare_verify(got, ref, n_nodes, bonus_margin=WALK_BONUS_MARGIN, walk=True)
    return ref, ex


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_configs(cfg):
    """The full workloads (trees, vocabularies, batch) in the bench's launch configuration."""
    ref, ex = _check(wl.config(cfg))
    print(f"cfg{cfg} walk: mean accept_len {ref['accept_len'].mean():.2f}, excused {ex}")


SMALL = [
    dict(B=16, N=37, V=5000),
    dict(B=8, N=63, V=2049, sigma_logits=1.0),
    dict(B=6, N=127, V=300, n_nodes_range=(1, 127), sigma_logits=0.5),
    dict(B=4, N=256, V=4099, tree=("random", 8)),
    dict(B=5, N=30, V=800, Vd=333),
    dict(B=9, N=10, V=1, tree=("random", 3)),
    dict(B=7, N=12, V=70000, draft_rows="per_depth", tree=("bfs", (3, 2, 2))),
    dict(B=6, N=40, V=3000, tree=("bfs", (12, 2, 1)), sigma_logits=0.7),     # wide sibling sets
    dict(B=4, N=64, V=20000, tree=("bfs", (63,)), sigma_logits=0.3),         # 63 siblings
    dict(B=5, N=40, V=7000, tree=("bfs", (1,) * 39)),                         # chains
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small(case):
    _check(wl.custom(seed=6000 + case, **SMALL[case]))


@pytest.mark.parametrize("parts,spin", [(2, None), (5, None), (16, None), (7, 1), (16, 1)])
def test_split_chain(tune, parts, spin):
    """A node's chain split over several workgroups (forced counts; at 16 some workgroups of a
    70000-token row have no step of it), and with a one-poll wait, on which workgroup 0 finishes
    the chain alone: the same decisions as the oracle.  Wide sibling sets (6, 3, 1 per level)
    give 14 nodes with several children, so 16 workgroups each still fit the GPU at once."""
    tune(walk_parts=parts, **({"walk_spin": spin} if spin else {}))
    w = wl.custom(seed=6200 + parts + (spin or 0), B=2, N=40, V=70000, tree=("bfs", (6, 3, 1)), sigma_logits=0.5)
    ref, ex = _check(w)
    print(f"walk_parts={parts} walk_spin={spin}: mean accept_len {ref['accept_len'].mean():.2f}, excused {ex}")


def test_split_chain_repeats(tune):
    """Twenty back-to-back runs of a split chain give bit-identical outputs: the partials of a
    pass are summed in a fixed order, and a workgroup one pass ahead writes the slots of the other
    parity (with one set of slots, a fast workgroup could overwrite a partial a sibling had not
    read yet, and the bonus token then moved)."""
    tune(walk_parts=16)
    w = wl.custom(seed=6216, B=2, N=40, V=70000, tree=("bfs", (6, 3, 1)), sigma_logits=0.5)
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    first, ref = _run(vi, parents, n_nodes, w.N - 1)
    compare_verify(first, ref, n_nodes, bonus_margin=WALK_BONUS_MARGIN, walk=True)
    for it in range(20):
        got = sb.spec_verify(dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents.astype(np.int32)),
                             dev(vi["uniforms"]), "walk", draft_probs=dev(vi["draft_probs"]),
                             draft_row=dev(vi["draft_row"]), n_nodes=dev(n_nodes.astype(np.int32)),
                             max_depth=w.N - 1)
        torch.cuda.synchronize()
        for k, v in got.items():
            assert np.array_equal(host(v), first[k]), (it, k)


def test_max_depth_and_errors():
    """Structural errors, a sibling on another draft row, and a tight max_depth."""
    w = wl.custom(seed=6100, B=12, N=30, V=900, tree=("random", 4))
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    tokens, draft_row, par = vi["tokens"].copy(), vi["draft_row"].copy(), parents.copy()
    par[0, 5] = 7                                   # parent after the child
    tokens[1, 3] = w.V                              # token out of range
    draft_row[2, 4] = vi["R"]                       # row out of range
    p2 = np.flatnonzero(np.bincount(par[3, 1:], minlength=w.N) >= 2)[0]   # a node with 2+ children
    kids = [c for c in range(1, w.N) if par[3, c] == p2]
    draft_row[3, kids[1]] = (draft_row[3, kids[0]] + 1) % vi["R"]   # sibling on another row
    n_nodes = n_nodes.copy()
    n_nodes[4] = w.N + 1                            # node count out of range
    n_nodes[5] = 0
    vi = dict(vi, tokens=tokens, draft_row=draft_row)
    for md in (w.N - 1, 2):
        got, ref = _run(vi, par, n_nodes, md)
        assert oracle.decode_err(ref["err"][3]) == (kids[1], oracle.ERR_DRAFTROW)
        assert (ref["err"] != 0).sum() >= 5
        compare_verify(got, ref, n_nodes, bonus_margin=WALK_BONUS_MARGIN, walk=True)


def test_chi_square_gpu():
    """The GPU walk emits the target's law on a branching tree with i.i.d. children (root with 3
    children, each with 2), where per-node rejection does not; and it agrees with the oracle on a
    slice of the same trials."""
    need_gpu()
    from scipy import stats as sps
    V, trials = 6, 100_000
    g = wl.rng(0, wl.S_TRIALS, 5151)
    L0 = (g.standard_normal(V) * 1.2).astype(np.float32)
    L2 = (g.standard_normal((V, V)) * 1.2).astype(np.float32)
    D = np.exp(g.standard_normal((2, V)))
    D = (D / D.sum(1, keepdims=True)).astype(np.float32)
    Dn = D.astype(np.float64) / D.astype(np.float64).sum(1, keepdims=True)
    par1 = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], np.int32)
    N = par1.size
    tokens = np.full((trials, N), -1, np.int32)
    tokens[:, 1:4] = g.choice(V, size=(trials, 3), p=Dn[0])
    tokens[:, 4:] = g.choice(V, size=(trials, 6), p=Dn[1])
    logits = np.empty((trials, N, V), np.float32)
    logits[:, 0] = L0
    for c in (1, 2, 3):
        logits[:, c] = L2[tokens[:, c]]
    logits[:, 4:] = 0.0
    u = g.random((trials, N), dtype=np.float32)
    parents = np.tile(par1, (trials, 1))
    dr = np.tile(np.array([-1, 0, 0, 0, 1, 1, 1, 1, 1, 1], np.int32), (trials, 1))
    draft = np.ascontiguousarray(np.broadcast_to(D, (trials, 2, V)))
    got = sb.spec_verify(dev(logits), dev(tokens), dev(parents), dev(u), "walk",
                         draft_probs=dev(draft), draft_row=dev(dr))
    torch.cuda.synchronize()
    acc, bonus, path = host(got["accept_len"]), host(got["bonus"]), host(got["path"])
    first = np.where(acc >= 1, tokens[np.arange(trials), np.maximum(path[:, 1], 0)], bonus)
    T0 = np.exp(L0.astype(np.float64)) / np.exp(L0.astype(np.float64)).sum()
    assert sps.chisquare(np.bincount(first, minlength=V), T0 * trials).pvalue > 1e-3
    sl = slice(0, 3000)
    ref = oracle.verify(logits[sl], tokens[sl], parents[sl], u[sl], oracle.MODE_WALK,
                        draft_probs=draft[sl], draft_row=dr[sl])
    gsl = {k: host(v)[sl] for k, v in got.items()}
    compare_verify(gsl, ref, np.full(3000, N), bonus_margin=WALK_BONUS_MARGIN, walk=True)
