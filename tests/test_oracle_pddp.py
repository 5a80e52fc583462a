"""Pins of the oracle's PDDP grouping (not gpu).

The MC-Sparse review (section 3) names Fast PDDP for equal-size, tile-aligned
query groups but prints no formula.  The oracle's reading (fixed-step power
iteration from the all-ones direction, rank split at floor(c/2)*G, ties to
the lower index, depth-first numbering) is pinned here against a textbook
eigensolver, closed-form special cases and the partition invariants.
"""
import numpy as np
import pytest

from oracle.mcs_oracle import (group_slices, pddp_groups, pddp_node_split, power_iteration,
                               tree_nodes)


def closed_form_iterate(C, T):
    """v_T = C^T v0 / ||C^T v0|| through the eigendecomposition of C."""
    lam, U = np.linalg.eigh(C)
    v0 = np.full(C.shape[0], 1.0 / np.sqrt(C.shape[0]))
    w = U @ ((lam / lam.max()) ** T * (U.T @ v0))
    return w / np.linalg.norm(w)


@pytest.mark.parametrize("d,T", [(4, 1), (8, 5), (16, 32), (64, 32), (128, 32)])
def test_power_iteration_equals_closed_form(d, T):
    rng = np.random.default_rng(d + T)
    X = rng.standard_normal((3 * d, d)) * np.linspace(0.3, 2.0, d)
    C = X.T @ X
    np.testing.assert_allclose(power_iteration(C, T), closed_form_iterate(C, T), rtol=0, atol=1e-10)


def test_power_iteration_converges_to_top_eigenvector_with_a_gap():
    rng = np.random.default_rng(11)
    d, T = 32, 32
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.concatenate([[10.0, 4.0], np.linspace(3.0, 0.1, d - 2)])   # lam2/lam1 = 0.4
    C = (U * lam) @ U.T
    v = power_iteration(C, T)
    u1 = U[:, 0]
    assert abs(abs(v @ u1) - 1.0) < 10 * 0.4 ** (2 * T) + 1e-12
    # sign is fixed by the all-ones start: <v, v0> >= 0
    assert v.sum() >= 0


def test_power_iteration_degenerate_keeps_start():
    v = power_iteration(np.zeros((6, 6)), 32)
    np.testing.assert_array_equal(v, np.full(6, 1 / np.sqrt(6)))


def test_hand_worked_two_way_split():
    # Points spread along x.  Worked by hand: mu = (5.5, 0.5), scatter
    # C = [[101, 10], [10, 1]], C v0 ~ (111, 11) so v ~ (0.995, 0.099);
    # projections of the four points are -5.52, 4.53, -4.53, 5.52, so the
    # left group (two smallest) is {0, 2}.
    Q = np.array([[0.0, 0.0], [10.0, 1.0], [1.0, 0.0], [11.0, 1.0]])
    assert pddp_groups(Q, G=2, iters=32).tolist() == [0, 2, 1, 3]
    # Mirror x: C = [[101, -10], [-10, 1]], C v0 ~ (91, -9), v ~ (0.995, -0.099);
    # projections 5.52, -4.53, 4.52, -5.52, so the left group is {1, 3}.
    Qm = Q * np.array([-1.0, 1.0])
    assert pddp_groups(Qm, G=2, iters=32).tolist() == [1, 3, 0, 2]


def test_hand_worked_split_needs_centering():
    # A large common offset along x, spread along y.  Centred: mu = (100, 5.5),
    # C = [[4, -2], [-2, 101]], principal direction ~ +y, so points split by y:
    # {0, 1} | {2, 3}.  Without centring the offset would dominate and split by x.
    Q = np.array([[101.0, 0.0], [99.0, 1.0], [101.0, 10.0], [99.0, 11.0]])
    assert pddp_groups(Q, G=2, iters=32).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("n,G", [(256, 64), (1000, 64), (777, 128), (64, 64), (65, 64), (3, 64)])
def test_rank_one_data_groups_are_sorted_runs(n, G):
    rng = np.random.default_rng(n)
    d = 16
    u = np.abs(rng.standard_normal(d)) + 0.1      # positive overlap with the all-ones start
    a = rng.permutation(n).astype(float) + 0.25 * rng.random(n)
    b = rng.standard_normal(d)
    Q = a[:, None] * u[None, :] + b[None, :]
    perm = pddp_groups(Q, G, 32)
    order = np.argsort(a, kind="stable")
    for s in group_slices(n, G):
        assert perm[s].tolist() == sorted(order[s].tolist())


def test_two_separated_clusters_never_share_a_group():
    rng = np.random.default_rng(21)
    G, d = 64, 32
    A = rng.standard_normal((3 * G, d)) + 25.0
    B = rng.standard_normal((5 * G, d)) - 25.0
    shuffle = rng.permutation(8 * G)
    Q = np.concatenate([A, B])[shuffle]
    inA = (np.arange(8 * G) < 3 * G)[shuffle]
    perm = pddp_groups(Q, G, 32)
    for s in group_slices(len(Q), G):
        assert len(set(inA[perm[s]].tolist())) == 1


@pytest.mark.parametrize("n,G", [(1024, 64), (4680, 64), (3000, 128), (130, 64), (1, 64), (64, 64)])
def test_partition_and_size_invariants(n, G):
    rng = np.random.default_rng(n + G)
    Q = rng.standard_normal((n, 8)) @ rng.standard_normal((8, 8))
    perm = pddp_groups(Q, G, 32)
    assert sorted(perm.tolist()) == list(range(n))
    sl = group_slices(n, G)
    sizes = [s.stop - s.start for s in sl]
    assert all(sz == G for sz in sizes[:-1]) and 1 <= sizes[-1] <= G
    for s in sl:
        assert np.all(np.diff(perm[s]) > 0)


def test_tree_nodes_are_contiguous_ranges_of_perm():
    rng = np.random.default_rng(5)
    n, G = 4680, 64
    Q = rng.standard_normal((n, 16))
    perm = pddp_groups(Q, G, 32)
    for level, start, size, c in tree_nodes(n, G):
        node = pddp_node_split(Q, np.sort(perm[start:start + size]), c, G, 32)
        nL = node["c_left"] * G
        assert node["left"].tolist() == sorted(perm[start:start + nL].tolist())
        assert node["right"].tolist() == sorted(perm[start + nL:start + size].tolist())
    # depth of the causal-chunk tree (74 groups): ragged, leaves at depth 6 and 7
    assert max(t[0] for t in tree_nodes(n, G)) == 6


def test_identical_queries_split_by_index():
    Q = np.tile(np.array([0.5, -1.0, 2.0]), (200, 1))
    perm = pddp_groups(Q, 64, 32)
    assert perm.tolist() == list(range(200))


def test_split_ties_broken_by_lower_index():
    # two exact duplicates straddle the split point; the lower index goes left
    Q = np.array([[0.0], [1.0], [1.0], [2.0]])
    node = pddp_node_split(Q, np.arange(4), 2, 2, 32)
    assert node["left"].tolist() == [0, 1] and node["right"].tolist() == [2, 3]
