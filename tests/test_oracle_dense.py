"""Pins of the oracle's dense attention (not gpu).

The pages print no worked values, so dense attention is pinned by its
definition written out as a pure-Python triple loop, by closed forms, and by
symmetries (softmax attention as used in every page's DiT; cost statement in
the FrameDiT summary, "1. 연구 배경").
"""
import math

import numpy as np
import pytest

from oracle.mcs_oracle import dense_attention, visible


def brute_dense(Q, K, V, scale, causal_block=0, q_offset=0):
    """Softmax attention by explicit loops over rows, keys and channels."""
    nq, nk, dv = len(Q), len(K), len(V[0])
    O = [[0.0] * dv for _ in range(nq)]
    lse = [0.0] * nq
    for i in range(nq):
        logits = []
        for j in range(nk):
            if causal_block and (j // causal_block) > ((q_offset + i) // causal_block):
                continue
            s = 0.0
            for c in range(len(Q[i])):
                s += Q[i][c] * K[j][c]
            logits.append((j, scale * s))
        m = max(l for _, l in logits)
        tot = sum(math.exp(l - m) for _, l in logits)
        lse[i] = m + math.log(tot)
        for j, l in logits:
            w = math.exp(l - m) / tot
            for c in range(dv):
                O[i][c] += w * V[j][c]
    return np.array(O), np.array(lse)


@pytest.mark.parametrize("nq,nk,d,scale,cb,qo", [
    (7, 11, 4, 0.5, 0, 0),
    (16, 16, 8, 1.3, 0, 0),
    (9, 30, 5, 0.8, 6, 12),     # frame-block causal, query chunk at the end
    (20, 20, 3, 2.0, 4, 0),     # causal self-attention with ragged blocks
])
def test_dense_matches_triple_loop(nq, nk, d, scale, cb, qo):
    rng = np.random.default_rng(nq * 1000 + nk)
    Q, K, V = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    O, lse = dense_attention(Q, K, V, scale, cb, qo, row_block=5)
    Ob, lseb = brute_dense(Q.tolist(), K.tolist(), V.tolist(), scale, cb, qo)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


def test_zero_queries_give_mean_of_visible_values():
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((24, 6)), rng.standard_normal((24, 6))
    Q = np.zeros((8, 6))
    O, lse = dense_attention(Q, K, V, 0.7)
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
    np.testing.assert_allclose(lse, np.log(24.0), atol=1e-14)
    # causal: query i (position 16 + i, blocks of 8) sees keys of blocks <= its own
    O, _ = dense_attention(Q, K, V, 0.7, causal_block=8, q_offset=16)
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
    O, _ = dense_attention(Q, K, V, 0.7, causal_block=8, q_offset=0)
    np.testing.assert_allclose(O, np.broadcast_to(V[:8].mean(0), O.shape), atol=1e-14)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(2)
    Q, K = rng.standard_normal((10, 4)), rng.standard_normal((13, 4))
    V = np.tile(np.array([1.5, -2.0, 0.25, 3.0]), (13, 1))
    O, _ = dense_attention(Q, K, V, 3.0, causal_block=5, q_offset=3)
    np.testing.assert_allclose(O, np.broadcast_to(V[0], O.shape), atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((5, 4)), rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    O, lse = dense_attention(Q, K, V, 1.0)
    np.testing.assert_allclose(O, np.broadcast_to(V[0], O.shape), atol=1e-15)
    np.testing.assert_allclose(lse, (Q @ K[0]), atol=1e-13)


def test_large_scale_selects_argmax():
    rng = np.random.default_rng(4)
    Q, K, V = rng.standard_normal((6, 5)), rng.standard_normal((9, 5)), rng.standard_normal((9, 5))
    O, _ = dense_attention(Q, K, V, 1e4)
    np.testing.assert_allclose(O, V[np.argmax(Q @ K.T, axis=1)], atol=1e-9)


def test_key_value_permutation_invariance_and_query_equivariance():
    rng = np.random.default_rng(5)
    Q, K, V = rng.standard_normal((12, 6)), rng.standard_normal((17, 6)), rng.standard_normal((17, 6))
    O, lse = dense_attention(Q, K, V, 0.9)
    pk = rng.permutation(17)
    O2, lse2 = dense_attention(Q, K[pk], V[pk], 0.9)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = rng.permutation(12)
    O3, lse3 = dense_attention(Q[pq], K, V, 0.9)
    np.testing.assert_allclose(O3, O[pq], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], atol=1e-13)


def test_causal_future_keys_do_not_matter_bitwise():
    rng = np.random.default_rng(6)
    blk, nk = 10, 50
    Q, K, V = rng.standard_normal((20, 4)), rng.standard_normal((nk, 4)), rng.standard_normal((nk, 4))
    q_offset = 20   # queries occupy blocks 2 and 3; keys of blocks 4.. are future
    O, lse = dense_attention(Q, K, V, 0.6, blk, q_offset)
    K2, V2 = K.copy(), V.copy()
    K2[40:] = rng.standard_normal((10, 4)) * 100
    V2[40:] = rng.standard_normal((10, 4)) * 100
    O2, lse2 = dense_attention(Q, K2, V2, 0.6, blk, q_offset)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_visibility_rule():
    v = visible(np.arange(4), np.arange(12), causal_block=3, q_offset=5)
    # query i at position 5+i -> block (5+i)//3 = 1,2,2,2 ; sees keys with j//3 <= that
    assert v[0].sum() == 6 and v[1].sum() == 9 and v[3].sum() == 9
    assert visible(np.arange(3), np.arange(5), 0, 0).all()


def test_rows_subset_and_row_blocks_agree():
    rng = np.random.default_rng(7)
    Q, K, V = rng.standard_normal((33, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    O, lse = dense_attention(Q, K, V, 0.4, 7, 2, row_block=4)
    rows = [0, 5, 32, 17]
    Os, lses = dense_attention(Q, K, V, 0.4, 7, 2, rows=rows)
    np.testing.assert_allclose(Os, O[rows], atol=1e-14)
    np.testing.assert_allclose(lses, lse[rows], atol=1e-14)
