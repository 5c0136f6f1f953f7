"""Pins of oracle.lm_head_stats: the logits against torch's float64 matmul, closed forms of the
row statistics (equal logits, two levels, a one-hot hidden state picking a column of W), the
entropy against scipy's entr, stability at large logits, the tie rule, the parent-row gather on
a hand-worked tree and the error rules."""

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_logits_match_library_matmul():
    rng = np.random.default_rng(1)
    h = bf16(rng.standard_normal((2, 5, 96)))
    W = bf16(rng.standard_normal((300, 96)) * 0.02)
    par = np.array([[-1, 0, 0, 1, 1], [-1, 0, 1, 2, 3]])
    tok = rng.integers(0, 300, size=(2, 5))
    r = oracle.lm_head_stats(h, W, par, tok)
    ref = torch.matmul(torch.from_numpy(h).double(), torch.from_numpy(W).double().T).numpy()
    assert np.allclose(r["logits"], ref, rtol=0, atol=1e-12)
    for b in range(2):
        for i in range(5):
            row = ref[b, i]
            assert r["row_max"][b, i] == row.max()
            assert r["row_argmax"][b, i] == int(np.argmax(row))
            e = np.exp(row - row.max())
            assert np.isclose(r["row_sum"][b, i], e.sum(), rtol=1e-13)
            # entropy of T from S and A against scipy's entr
            H = np.log(r["row_sum"][b, i]) - r["row_ent"][b, i] / r["row_sum"][b, i]
            assert np.isclose(H, scipy.special.entr(e / e.sum()).sum(), rtol=1e-11)


def test_closed_forms():
    # all logits equal: S = V, A = 0, argmax = 0 (lowest id on ties)
    m, am, S, A = oracle.row_statistics(np.full(1000, 3.25))
    assert (m, am, S, A) == (3.25, 0, 1000.0, 0.0)
    # two levels: n1 at a, n2 at a - d  =>  S = n1 + n2 e^-d, A = -n2 d e^-d
    row = np.array([5.0] * 3 + [5.0 - 2.0] * 7)
    m, am, S, A = oracle.row_statistics(row[::-1].copy())
    assert m == 5.0 and am == 7
    assert np.isclose(S, 3 + 7 * np.exp(-2.0), rtol=1e-15)
    assert np.isclose(A, -7 * 2.0 * np.exp(-2.0), rtol=1e-15)
    # large logits stay finite (the maximum is subtracted before exponentiating)
    m, am, S, A = oracle.row_statistics(np.array([1000.0, 999.0, 2000.0, 2000.0]))
    assert (m, am) == (2000.0, 2) and S == 2.0 and A == 0.0


def test_one_hot_hidden_picks_a_column_of_W():
    """h_i = e_j gives l_i = W[:, j]: the statistics of a known column, and the gathers read
    the parent's row, not the child's."""
    rng = np.random.default_rng(4)
    V, Dm = 50, 8
    W = bf16(rng.standard_normal((V, Dm)))
    h = np.zeros((1, 4, Dm), dtype=np.float32)
    cols = [3, 0, 7, 5]
    for i, j in enumerate(cols):
        h[0, i, j] = 1.0
    par = np.array([[-1, 0, 0, 2]])
    tok = np.array([[-1, 11, 42, 9]])
    r = oracle.lm_head_stats(h, W, par, tok)
    for i, j in enumerate(cols):
        col = W[:, j].astype(np.float64)
        assert r["row_max"][0, i] == col.max() and r["row_argmax"][0, i] == int(np.argmax(col))
    assert np.isnan(r["cand_logit"][0, 0])
    assert r["cand_logit"][0, 1] == W[11, cols[0]]       # parent 0 looks at column 3
    assert r["cand_logit"][0, 2] == W[42, cols[0]]
    assert r["cand_logit"][0, 3] == W[9, cols[2]]        # parent 2 looks at column 7


def test_ties_and_square_orientation():
    """A square W distinguishes W h from W^T h; equal maxima go to the lower id."""
    W = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 2.0], [0.0, 0.0, 2.0]], dtype=np.float32)
    h = np.array([[[0.0, 0.0, 1.0]]], dtype=np.float32)
    r = oracle.lm_head_stats(h, W, np.array([[-1]]), np.array([[-1]]))
    assert r["logits"][0, 0].tolist() == [0.0, 2.0, 2.0]      # W h (W^T h would be [0, 0, 4])
    assert r["row_argmax"][0, 0] == 1


def test_ragged_and_errors():
    rng = np.random.default_rng(2)
    h = bf16(rng.standard_normal((5, 4, 16)))
    W = bf16(rng.standard_normal((40, 16)))
    par = np.tile(np.array([-1, 0, 0, 1]), (5, 1))
    tok = np.tile(np.array([-1, 3, 39, 0]), (5, 1))
    par[1, 0] = 0
    par[2, 3] = 3
    tok[3, 2] = 40
    n = np.array([2, 4, 4, 4, 5])
    r = oracle.lm_head_stats(h, W, par, tok, n_nodes=n)
    assert [oracle.decode_err(e) for e in r["err"]] == [(0, 0), (0, oracle.ERR_ROOT), (3, oracle.ERR_PARENT),
                                                         (2, oracle.ERR_TOKEN), (0, oracle.ERR_NNODES)]
    assert np.isfinite(r["row_max"][0, :2]).all() and np.isnan(r["row_max"][0, 2:]).all()
    assert (r["row_argmax"][1:] == -1).all() and np.isnan(r["cand_logit"][1:]).all()
