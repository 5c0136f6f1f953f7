"""GPU parity: spec_kv_compact against the oracle, bit-exact (the operation copies slots).  Paths
come from spec_verify on seeded trees (chains and branching trees), with error words and invalid
paths mixed in; a long path exercises many copy passes; two rounds run back to back on the
device, the second on the first's compacted cache and prefix lengths."""

import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_spec_amd import binding as sb
from tree_attention_verification_spec_amd import workloads as wl

from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _caches(rng, L, B, H, S, d, dtype):
    k = rng.standard_normal((L, B, H, S, d)).astype(np.float32)
    v = rng.standard_normal((L, B, H, S, d)).astype(np.float32)
    if dtype == torch.bfloat16:
        k, v = wl.round_bf16(k), wl.round_bf16(v)
    return k, v


def _verify_paths(seed, B, N, V, tree, mode="reject"):
    w = wl.custom(seed=seed, B=B, N=N, V=V, tree=tree)
    parents, n_nodes = wl.trees(w)
    vi = wl.verify_inputs(w, parents)
    ref = oracle.verify(vi["target_logits"], vi["tokens"], parents, vi["uniforms"],
                        {"greedy": oracle.MODE_GREEDY, "reject": oracle.MODE_REJECT}[mode],
                        draft_probs=vi["draft_probs"], draft_row=vi["draft_row"], t2d=vi["t2d"],
                        n_nodes=n_nodes, eps=0.09, delta=0.3, max_depth=N - 1)
    return ref["path"].astype(np.int32), ref["accept_len"].astype(np.int32), ref["err"].astype(np.int32)


def _run(k, v, P, path, acc, err, dtype, four_d=False):
    need_gpu()
    kd = torch.from_numpy(k).to(dtype).cuda()
    vd = torch.from_numpy(v).to(dtype).cuda()
    if four_d:
        kd, vd = kd[0].contiguous(), vd[0].contiguous()
    Pout = sb.spec_kv_compact(kd, vd, dev(P.astype(np.int32)), dev(path), dev(acc),
                              err=None if err is None else dev(err))
    torch.cuda.synchronize()
    if four_d:
        kd, vd = kd[None], vd[None]
    return kd.float().cpu().numpy(), vd.float().cpu().numpy(), host(Pout)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tree", [("random", 6), ("bfs", (1,) * 39), ("bfs", (4, 3, 2))])
def test_paths_from_verify(dtype, d, tree):
    B, N, H, L = 6, 40, 4, 3
    path, acc, err = _verify_paths(4000 + d, B, N, 64, tree)
    rng = np.random.default_rng(7)
    P = rng.integers(0, 30, size=B)
    S = int(P.max()) + N + 3
    k, v = _caches(rng, L, B, H, S, d, dtype)
    # mix in: a verification error, and a path that is not increasing
    err = err.copy()
    err[1] = (3 << 8) | 2
    if acc[4] >= 2:
        path = path.copy()
        path[4, 1], path[4, 2] = path[4, 2], path[4, 1]
    kg, vg, Pg = _run(k, v, P, path, acc, err, dtype)
    kr, vr, Pr = oracle.kv_compact(k, v, P, path, acc, err)
    assert np.array_equal(Pg, Pr)
    assert np.array_equal(kg, kr) and np.array_equal(vg, vr)


def test_long_path_and_single_layer():
    """A 200-deep path (many passes of a wave's copy loop) with gaps, in a one-layer (4-D) cache,
    and out-of-cache / negative-length sequences left untouched."""
    B, H, S, d, md = 4, 2, 700, 128, 255
    rng = np.random.default_rng(11)
    k, v = _caches(rng, 1, B, H, S, d, torch.bfloat16)
    path = np.full((B, md + 1), -1, dtype=np.int32)
    nodes = np.sort(rng.choice(np.arange(1, 400), size=200, replace=False))
    path[0, 0], path[0, 1:201] = 0, nodes
    path[1, :4] = [0, 2, 3, 5]
    path[2, :3] = [0, 10, 690]                  # P + 690 past the cache
    path[3, :2] = [0, 1]
    acc = np.array([200, 3, 2, -1], dtype=np.int32)
    P = np.array([50, 0, 40, 7])
    kg, vg, Pg = _run(k, v, P, path, acc, None, torch.bfloat16, four_d=True)
    kr, vr, Pr = oracle.kv_compact(k, v, P, path, acc)
    assert Pg.tolist() == Pr.tolist() == [251, 4, 40, 7]
    assert np.array_equal(kg, kr) and np.array_equal(vg, vr)


def test_two_rounds_on_the_device():
    """verify -> compact -> verify -> compact with every intermediate kept on the GPU; the oracle
    replays the same two rounds on the GPU's verification outputs."""
    need_gpu()
    B, N, H, L, d = 5, 30, 2, 2, 64
    rng = np.random.default_rng(5)
    P0 = rng.integers(0, 20, size=B)
    S = int(P0.max()) + 2 * (N + 2)
    k, v = _caches(rng, L, B, H, S, d, torch.float32)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    Pd = dev(P0.astype(np.int32))
    kr, vr, Pr = k, v, P0.astype(np.int32)
    for rnd in range(2):
        w = wl.custom(seed=4100 + rnd, B=B, N=N, V=80, tree=("random", 5))
        parents, n_nodes = wl.trees(w)
        vi = wl.verify_inputs(w, parents)
        got = sb.spec_verify(dev(vi["target_logits"]), dev(vi["tokens"]), dev(parents.astype(np.int32)),
                             dev(vi["uniforms"]), "reject", draft_probs=dev(vi["draft_probs"]),
                             draft_row=dev(vi["draft_row"]), n_nodes=dev(n_nodes.astype(np.int32)),
                             max_depth=N - 1)
        Pd = sb.spec_kv_compact(kd, vd, Pd, got["path"], got["accept_len"], err=got["err"])
        torch.cuda.synchronize()
        kr, vr, Pr = oracle.kv_compact(kr, vr, Pr, host(got["path"]), host(got["accept_len"]), host(got["err"]))
        assert np.array_equal(host(Pd), Pr)
        assert np.array_equal(kd.cpu().numpy(), kr) and np.array_equal(vd.cpu().numpy(), vr)
