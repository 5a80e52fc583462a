"""Pins of the oracle's block-sparse comparator (not gpu).

MC-Sparse review, sections 1 and 2: block-sparse attention scores KV blocks
approximately (mean pooling) and keeps whole blocks.  Pins: a hand-worked
example (scores, tie order, the partial last block, a causal limit), the
special case of 1-token blocks and 1-query groups (an exact per-query sort of
the logits), ranking consistency against block-averaged exact logits
(bilinearity: <mean q, mean k> is the mean of the block's logits), and the
full-budget case (every token kept: block-sparse equals dense attention).
"""
import numpy as np
import pytest

from oracle.mcs_oracle import block_pooled_selection, block_sparse_step, dense_attention


def hand_case():
    # 4 KV blocks of 2 keys in d = 2: means (1,0), (0,2), (4,0), (0,-1)
    K = np.array([[1, 0], [1, 0], [0, 1], [0, 3], [5, 0], [3, 0], [0, -1], [0, -1]], dtype=float)
    # one group of 2 queries with mean (1, 1): scores 1, 2, 4, -1
    Q = np.array([[2, 0], [0, 2]], dtype=float)
    return Q, K


@pytest.mark.parametrize("k,expect", [
    (1, [4]),                      # best block (2), its lowest token
    (3, [2, 4, 5]),                # block 2, then one token of block 1
    (4, [2, 3, 4, 5]),
    (5, [0, 2, 3, 4, 5]),          # then block 0 (score 1), lowest token first
    (7, [0, 1, 2, 3, 4, 5, 6]),    # block 3 (score -1) last
    (8, list(range(8))),
])
def test_hand_example(k, expect):
    Q, K = hand_case()
    assert block_pooled_selection(Q, K, G=2, k=k, scale=1.0, block=2)[0].tolist() == expect


def test_hand_example_ties_go_to_the_lower_block():
    Q, K = hand_case()
    K = K.copy()
    K[4:6] = [[1, 0], [1, 0]]      # block 2 now ties block 0 (score 1)
    # order: block 1 (2), block 0 (1), block 2 (1), block 3
    assert block_pooled_selection(Q, K, 2, 3, 1.0, block=2)[0].tolist() == [0, 2, 3]
    assert block_pooled_selection(Q, K, 2, 5, 1.0, block=2)[0].tolist() == [0, 1, 2, 3, 4]


def test_hand_example_causal_limit():
    Q, K = hand_case()
    # queries at positions 2 and 3, frames of 2 tokens: keys 0..3 visible (blocks 0 and 1)
    sel = block_pooled_selection(Q, K, 2, 3, 1.0, causal_block=2, q_offset=2, block=2)
    assert sel[0].tolist() == [0, 2, 3]        # block 2 (score 4) is not visible
    # more than the visible tokens: invisible blocks follow in index order
    sel = block_pooled_selection(Q, K, 2, 6, 1.0, causal_block=2, q_offset=2, block=2)
    assert sel[0].tolist() == [0, 1, 2, 3, 4, 5]


def test_ragged_last_blocks():
    Q, K = hand_case()
    K = K[:7]                      # last block holds one key (mean (0,-1))
    Q3 = np.vstack([Q, [[1.0, 1.0]]])   # groups of 2: {0,1} and {2}
    sel = block_pooled_selection(Q3, K, 2, 7, 1.0, block=2)
    assert sel.tolist() == [list(range(7)), list(range(7))]
    sel = block_pooled_selection(Q3, K, 2, 6, 1.0, block=2)
    # both groups have mean (1,1): blocks 2, 1, 0 fill exactly 6 tokens
    assert sel.tolist() == [[0, 1, 2, 3, 4, 5]] * 2


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_unit_blocks_and_groups_give_an_exact_per_query_sort(seed):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((5, 8))
    K = rng.standard_normal((40, 8))
    K[7] = K[3]                    # an exact tie in every row
    k = 7
    sel = block_pooled_selection(Q, K, G=1, k=k, scale=0.37, block=1)
    for i in range(5):
        logits = [float(np.dot(Q[i], K[j])) for j in range(40)]
        ranked = sorted(range(40), key=lambda j: (-logits[j], j))
        assert sel[i].tolist() == sorted(ranked[:k])


@pytest.mark.parametrize("seed,Nq,Nkv,G,k,block", [(0, 200, 333, 64, 90, 16), (1, 130, 257, 64, 64, 64),
                                                   (2, 256, 200, 128, 33, 8)])
def test_selection_is_whole_blocks_ranked_by_mean_logit(seed, Nq, Nkv, G, k, block):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Nq, 16))
    K = rng.standard_normal((Nkv, 16)) + 0.3 * rng.standard_normal(16)
    scale = 0.25
    sel = block_pooled_selection(Q, K, G, k, scale, block=block)
    nkb = -(-Nkv // block)
    for g in range(-(-Nq // G)):
        rows = slice(g * G, min((g + 1) * G, Nq))
        s = sel[g]
        assert len(set(s.tolist())) == k and np.all(np.diff(s) > 0)
        # block scores from the exact logits: the mean over the block pair
        L = scale * Q[rows] @ K.T
        score = np.array([L[:, b * block:(b + 1) * block].mean() for b in range(nkb)])
        taken = np.bincount(s // block, minlength=nkb)
        size = np.array([min(block, Nkv - b * block) for b in range(nkb)])
        whole = np.flatnonzero(taken == size)
        part = np.flatnonzero((taken > 0) & (taken < size))
        none = np.flatnonzero(taken == 0)
        assert len(part) <= 1
        for b in part:                          # the lowest tokens of the partial block
            assert s[s // block == b].tolist() == list(range(b * block, b * block + taken[b]))
        lo = score[whole].min() if len(whole) else np.inf
        hi = score[none].max() if len(none) else -np.inf
        assert lo >= hi - 1e-12
        for b in part:
            assert score[b] <= lo + 1e-12 and score[b] >= hi - 1e-12


def test_full_budget_keeps_every_token_and_equals_dense():
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((150, 16))
    K = rng.standard_normal((130, 16))
    V = rng.standard_normal((130, 16))
    perm, idx, O = block_sparse_step(Q, K, V, 64, 130, 0.25, causal_block=50, q_offset=10)
    assert perm.tolist() == list(range(150))
    assert all(row.tolist() == list(range(130)) for row in idx)
    Od, _ = dense_attention(Q, K, V, 0.25, 50, 10)
    assert np.abs(O - Od).max() < 1e-12
