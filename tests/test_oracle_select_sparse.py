"""Pins of the oracle's column mass, top-k selection, sparse attention and residual (not gpu).

MC-Sparse review, section 3: exact per-group attention scores at an anchor,
token-level KV selection, R = O_full - O_sparse added back on reuse steps.
Pins: explicit-loop definitions, conservation (rows of P sum to one),
order statistics, and the identities that hold by the method's construction
(keep 100% means sparse equals dense; zero drift means the reuse step returns
the anchor's dense output).
"""
import math

import numpy as np
import pytest

from oracle.mcs_oracle import (anchor_step, column_mass, dense_attention, group_slices, pddp_groups,
                               reuse_step, sparse_attention, topk_select)


def brute_topk(m, k):
    """Repeatedly take the largest remaining mass, lowest index first."""
    left = list(range(len(m)))
    out = []
    for _ in range(k):
        best = left[0]
        for j in left[1:]:
            if m[j] > m[best]:
                best = j
        out.append(best)
        left.remove(best)
    return sorted(out)


@pytest.mark.parametrize("n,k,seed", [(20, 5, 0), (31, 1, 1), (31, 31, 2), (64, 10, 3), (50, 17, 4)])
def test_topk_matches_selection_by_loops_with_ties(n, k, seed):
    rng = np.random.default_rng(seed)
    m = rng.integers(0, 6, n).astype(float) / 4.0      # many exact ties
    assert topk_select(m, k).tolist() == brute_topk(m.tolist(), k)


def test_topk_order_statistics():
    rng = np.random.default_rng(9)
    m = rng.random(1000) ** 3
    m[[5, 600, 700]] = m[100]                        # ties
    k = 137
    sel = topk_select(m, k)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    unsel = np.setdiff1d(np.arange(1000), sel)
    assert m[sel].min() >= m[unsel].max()
    t = m[sel].min()
    # among keys whose mass equals the threshold, the selected ones are the lowest indices
    tied = np.flatnonzero(m == t)
    chosen = np.intersect1d(tied, sel)
    assert np.all(chosen[:, None] < np.setdiff1d(tied, sel)[None, :])


def brute_mass(Q, K, lse, members, scale, cb, qo):
    m = [0.0] * len(K)
    for i in members:
        for j in range(len(K)):
            if cb and j // cb > (qo + i) // cb:
                continue
            s = sum(Q[i][c] * K[j][c] for c in range(len(Q[i])))
            m[j] += math.exp(scale * s - lse[i])
    return np.array(m)


@pytest.mark.parametrize("cb,qo", [(0, 0), (5, 10)])
def test_column_mass_matches_loops_and_conserves_rows(cb, qo):
    rng = np.random.default_rng(cb)
    Q, K, V = rng.standard_normal((12, 4)), rng.standard_normal((25, 4)), rng.standard_normal((25, 4))
    _, lse = dense_attention(Q, K, V, 0.8, cb, qo)
    members = np.array([1, 4, 7, 10])
    m = column_mass(Q, K, lse, members, 0.8, cb, qo)
    np.testing.assert_allclose(m, brute_mass(Q.tolist(), K.tolist(), lse, members, 0.8, cb, qo),
                               atol=1e-13)
    assert np.all(m >= 0)
    np.testing.assert_allclose(m.sum(), len(members), atol=1e-12)


def brute_sparse_row(q, K, V, sel, scale, vis):
    terms = [(j, scale * float(np.dot(q, K[j]))) for j in sel if vis(j)]
    if not terms:
        return np.zeros(V.shape[1])
    mx = max(t for _, t in terms)
    z = sum(math.exp(t - mx) for _, t in terms)
    return sum(math.exp(t - mx) / z * V[j] for j, t in terms)


@pytest.mark.parametrize("cb,qo", [(0, 0), (6, 12)])
def test_sparse_matches_renormalised_loops(cb, qo):
    rng = np.random.default_rng(40 + cb)
    nq, nk, G, k = 10, 30, 4, 7
    Q, K, V = rng.standard_normal((nq, 5)), rng.standard_normal((nk, 5)), rng.standard_normal((nk, 5))
    perm = rng.permutation(nq)
    for s in group_slices(nq, G):
        perm[s] = np.sort(perm[s])
    idx = np.stack([np.sort(rng.choice(nk, k, replace=False)) for _ in group_slices(nq, G)])
    O = sparse_attention(Q, K, V, perm, idx, G, 0.7, cb, qo)
    for g, s in enumerate(group_slices(nq, G)):
        for i in perm[s]:
            vis = (lambda j, i=i: (cb == 0) or (j // cb <= (qo + i) // cb))
            np.testing.assert_allclose(O[i], brute_sparse_row(Q[i], K, V, idx[g], 0.7, vis), atol=1e-13)


def test_sparse_row_without_visible_selection_is_zero():
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((2, 3)), rng.standard_normal((20, 3)), rng.standard_normal((20, 3))
    # both queries in block 0 (positions 0,1; blocks of 5); selection only future keys
    O = sparse_attention(Q, K, V, np.array([0, 1]), np.array([[10, 15, 19]]), 2, 1.0, 5, 0)
    assert np.array_equal(O, np.zeros_like(O))


def test_single_selected_key_returns_its_value():
    rng = np.random.default_rng(4)
    Q, K, V = rng.standard_normal((4, 3)), rng.standard_normal((9, 3)), rng.standard_normal((9, 3))
    O = sparse_attention(Q, K, V, np.arange(4), np.array([[6], [2]]), 2, 1.0)
    np.testing.assert_allclose(O[:2], np.broadcast_to(V[6], (2, 3)), atol=1e-15)
    np.testing.assert_allclose(O[2:], np.broadcast_to(V[2], (2, 3)), atol=1e-15)


@pytest.mark.parametrize("cb,qo,nq,nk", [(0, 0, 200, 200), (50, 150, 100, 250)])
def test_full_keep_makes_sparse_equal_dense_and_residual_vanish(cb, qo, nq, nk):
    rng = np.random.default_rng(nq)
    Q, K, V = rng.standard_normal((nq, 8)), rng.standard_normal((nk, 8)), rng.standard_normal((nk, 8))
    a = anchor_step(Q, K, V, G=64, k=nk, scale=0.5, causal_block=cb, q_offset=qo, iters=32)
    assert all(a["idx"][g].tolist() == list(range(nk)) for g in range(a["idx"].shape[0]))
    O_sp = sparse_attention(Q, K, V, a["perm"], a["idx"], 64, 0.5, cb, qo)
    np.testing.assert_allclose(O_sp, a["O_full"], atol=1e-13)
    assert np.abs(a["R"]).max() < 1e-13


@pytest.mark.parametrize("cb,qo", [(0, 0), (64, 128)])
def test_anchor_identity_and_zero_drift_reuse(cb, qo):
    rng = np.random.default_rng(77)
    nq, nk, G, k = 192, 300, 64, 30
    Q, K, V = rng.standard_normal((nq, 16)), rng.standard_normal((nk, 16)), rng.standard_normal((nk, 16))
    a = anchor_step(Q, K, V, G, k, 0.3, cb, qo, 32)
    O_sp = sparse_attention(Q, K, V, a["perm"], a["idx"], G, 0.3, cb, qo)
    np.testing.assert_allclose(O_sp + a["R"], a["O_full"], atol=1e-14)
    O = reuse_step(Q, K, V, a["perm"], a["idx"], a["R"], G, 0.3, cb, qo)
    np.testing.assert_allclose(O, a["O_full"], atol=1e-14)
    # the selection really is sparse: the residual is not negligible here
    assert np.abs(a["R"]).max() > 1e-3
    # each group's selection is its exact top-k by column mass
    for g, s in enumerate(group_slices(nq, G)):
        m = column_mass(Q, K, a["lse"], a["perm"][s], 0.3, cb, qo)
        assert a["idx"][g].tolist() == brute_topk(m.tolist(), k)


def test_reuse_adds_residual_to_sparse_output():
    rng = np.random.default_rng(8)
    nq, nk, G, k = 128, 128, 64, 16
    Q, K, V = rng.standard_normal((nq, 8)), rng.standard_normal((nk, 8)), rng.standard_normal((nk, 8))
    perm = pddp_groups(Q, G, 32)
    idx = np.stack([np.arange(k), np.arange(k) + 50])
    R = rng.standard_normal((nq, 8))
    O = reuse_step(Q, K, V, perm, idx, R, G, 1.0)
    np.testing.assert_allclose(O - R, sparse_attention(Q, K, V, perm, idx, G, 1.0), atol=1e-14)


# --- residual-drift check (adaptive anchoring) ------------------------------
from oracle.mcs_oracle import sampled_drift  # noqa: E402


def test_drift_on_all_rows_is_the_relative_error():
    rng = np.random.default_rng(21)
    Q, K, V = rng.standard_normal((40, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    Od, _ = dense_attention(Q, K, V, 0.4, 10, 5)
    O = Od + 0.01 * rng.standard_normal(Od.shape)
    rel = np.linalg.norm(O - Od) / np.linalg.norm(Od)
    assert abs(sampled_drift(O, Q, K, V, np.arange(40), 0.4, 10, 5) - rel) < 1e-12
    assert sampled_drift(Od, Q, K, V, [3, 17, 39], 0.4, 10, 5) < 1e-14


def test_drift_hand_example():
    # two keys, equal logits for row 0: exact output = mean of the values
    Q = np.array([[0.0, 0.0], [1.0, 0.0]])
    K = np.array([[1.0, 0.0], [-1.0, 0.0]])
    V = np.array([[2.0, 0.0], [0.0, 2.0]])
    O = np.array([[1.0, 1.0 + 0.3], [9.0, 9.0]])
    # row 0 exact (1, 1): error 0.3, norm sqrt(2)
    assert abs(sampled_drift(O, Q, K, V, [0], 1.0) - 0.3 / math.sqrt(2.0)) < 1e-12
    # causal frames of one token: row 0 at position 0 sees key 0 only -> exact (2, 0)
    assert abs(sampled_drift(O, Q, K, V, [0], 1.0, causal_block=1) - math.hypot(1.0, 1.3) / 2.0) < 1e-12


def test_drift_of_the_reuse_output_is_the_residual_movement():
    """At the anchor step itself the reuse output is the dense output (drift 0);
    on a later step it is |R_anchor - R_now| relative to the output."""
    rng = np.random.default_rng(22)
    Q, K, V = rng.standard_normal((130, 8)), rng.standard_normal((130, 8)), rng.standard_normal((130, 8))
    a = anchor_step(Q, K, V, 64, 20, 0.5, iters=8)
    rows = np.arange(0, 130, 7)
    O0 = reuse_step(Q, K, V, a["perm"], a["idx"], a["R"], 64, 0.5)
    assert sampled_drift(O0, Q, K, V, rows, 0.5) < 1e-12
    Q1, K1, V1 = (x + 0.1 * rng.standard_normal(x.shape) for x in (Q, K, V))
    O1 = reuse_step(Q1, K1, V1, a["perm"], a["idx"], a["R"], 64, 0.5)
    Od1, _ = dense_attention(Q1, K1, V1, 0.5)
    R_now = Od1 - sparse_attention(Q1, K1, V1, a["perm"], a["idx"], 64, 0.5)
    want = np.linalg.norm((a["R"] - R_now)[rows]) / np.linalg.norm(Od1[rows])
    assert abs(sampled_drift(O1, Q1, K1, V1, rows, 0.5) - want) < 1e-12
