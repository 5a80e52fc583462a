"""Independent fp64 CPU oracle of MC-Sparse token-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.  It shares no code, constants or helpers with the HIP
path and is deliberately plain: numpy in float64, one head at a time, dense
work in row blocks so that no Nq x Nkv matrix is ever held.

Source of the method: the review page "[논문리뷰] MC-Sparse: Deconstructing and
Closing the Dense-Sparse Attention Gap in Diffusion Transformers"
(blog.secrett2633.cloud), section "3. Method & Key Results".  It describes:
  * per-query-group selection of individual KV tokens, not blocks;
  * equal-size, tile-aligned query groups of similar queries built by
    Fast Principal Direction Divisive Partitioning (PDDP);
  * exact attention scores computed at an anchor step, whose KV selections
    are reused on the following steps;
  * a residual R = O_full - O_sparse taken at the anchor and added back on the
    reuse steps as an additive correction.
The page gives no formulas, so where it is silent this module takes the
plainest reading (documented per function).  The dense attention it
approximates is ordinary softmax attention over all (visible) 3D tokens, whose
quadratic cost is the bottleneck stated in the FrameDiT summary (gist.science,
"1. 연구 배경") and in the MC-Sparse review (section 2, motivation).

Conventions: one head per call; Q [Nq, d], K and V [Nkv, d] as float64 (the
inputs are the exact bf16/fp32 values the GPU consumes).  Query row i sits at
position ``q_offset + i`` of the KV sequence.  With ``causal_block == 0``
every key is visible; otherwise key j is visible to query i iff
floor(j / causal_block) <= floor((q_offset + i) / causal_block)
(frame-block causal attention for chunked video generation).

Parity of the method as a whole against the pages' published quality numbers
(PSNR, speedups) is unpinned: those need the paper's models.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

_F = np.float64


def _as64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=_F)


# ---------------------------------------------------------------------------
# Visibility
# ---------------------------------------------------------------------------
def visible(q_rows: np.ndarray, keys: np.ndarray, causal_block: int, q_offset: int) -> np.ndarray:
    """Boolean [len(q_rows), len(keys)]: may query row i attend to key j.

    Frame-block causal masking (a query frame sees its own and earlier
    frames); everything is visible when ``causal_block`` is 0.
    """
    q_rows = np.asarray(q_rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    if causal_block == 0:
        return np.ones((q_rows.size, keys.size), dtype=bool)
    qb = (q_offset + q_rows) // causal_block
    kb = keys // causal_block
    return kb[None, :] <= qb[:, None]


# ---------------------------------------------------------------------------
# Dense attention (the output MC-Sparse approximates)
# ---------------------------------------------------------------------------
def dense_attention(Q, K, V, scale: float, causal_block: int = 0, q_offset: int = 0,
                    rows: Optional[Sequence[int]] = None, row_block: int = 1024
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention O_i = sum_j P_ij v_j with P_ij = exp(l_ij - lse_i).

    l_ij = scale * <q_i, k_j> over visible j; lse_i = log sum_j exp(l_ij)
    (natural log).  Returns (O [n, d], lse [n]) for the requested rows (all
    rows by default).  A row with no visible key gets O = 0, lse = -inf.
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, V.shape[1]), _F)
    lse = np.full(rows.size, -np.inf, _F)
    keys = np.arange(K.shape[0])
    for s in range(0, rows.size, row_block):
        r = rows[s:s + row_block]
        logits = scale * (Q[r] @ K.T)
        vis = visible(r, keys, causal_block, q_offset)
        logits = np.where(vis, logits, -np.inf)
        mx = logits.max(axis=1)
        ok = np.isfinite(mx)
        safe_mx = np.where(ok, mx, 0.0)
        E = np.exp(logits - safe_mx[:, None])
        den = E.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            P = np.where(ok[:, None], E / np.where(ok, den, 1.0)[:, None], 0.0)
            lse[s:s + r.size] = np.where(ok, safe_mx + np.log(np.where(ok, den, 1.0)), -np.inf)
        O[s:s + r.size] = P @ V
    return O, lse


# ---------------------------------------------------------------------------
# PDDP query grouping
# ---------------------------------------------------------------------------
def power_iteration(C: np.ndarray, iters: int) -> np.ndarray:
    """Principal direction of a symmetric PSD matrix by a fixed number of steps.

    v_0 = (1, ..., 1) / sqrt(d);  v_{t+1} = C v_t / ||C v_t||_2.  A step whose
    product is exactly zero keeps v_t (degenerate node, all members equal).
    The fixed start and step count make the direction a deterministic function
    of C (v_T is proportional to C^T v_0, with its sign fixed by v_0).
    """
    C = _as64(C)
    d = C.shape[0]
    v = np.full(d, 1.0 / np.sqrt(d))
    for _ in range(iters):
        w = C @ v
        nrm = np.sqrt(w @ w)
        if nrm == 0.0:
            break
        v = w / nrm
    return v


def pddp_node_split(Q, members: np.ndarray, n_groups: int, G: int, iters: int):
    """One PDDP bisection of a node (the "Fast PDDP" step of the MC-Sparse review, section 3).

    The node's queries are centred on their mean, projected on the principal
    direction of their scatter matrix, and ranked by (projection, original
    index).  The first floor(c/2)*G of that ranking form the left child and the
    rest the right child, so every left child holds a whole number of groups
    ("equal-size, tile-aligned").

    Returns dict with left/right member arrays (ascending), child group counts,
    the projections p (aligned with ``members``), the ranking, the direction
    and the split point (midpoint of the n_L-th and (n_L+1)-th ranked
    projections).
    """
    Q = _as64(Q)
    members = np.asarray(members, dtype=np.int64)
    X = Q[members]
    mu = X.mean(axis=0)
    Xc = X - mu
    C = Xc.T @ Xc
    v = power_iteration(C, iters)
    p = Xc @ v
    order = np.lexsort((members, p))          # by p, then by original index
    cL = n_groups // 2
    nL = cL * G
    left = np.sort(members[order[:nL]])
    right = np.sort(members[order[nL:]])
    ranked = p[order]
    split_point = 0.5 * (ranked[nL - 1] + ranked[nL])
    return {"left": left, "right": right, "c_left": cL, "c_right": n_groups - cL,
            "p": p, "order": order, "v": v, "mu": mu, "split_point": split_point}


def pddp_groups(Q, G: int, iters: int) -> np.ndarray:
    """PDDP grouping of one head's queries into ceil(Nq/G) groups.

    Recursive balanced bisection (``pddp_node_split``) until a node holds one
    group; groups are numbered in depth-first (left-first) order and listed
    contiguously.  Returns ``perm`` [Nq]: perm[g*G : (g+1)*G] are the members
    of group g in ascending original index.  Only the last group may be short.
    """
    Q = _as64(Q)
    Nq = Q.shape[0]
    out: List[np.ndarray] = []

    def split(members: np.ndarray, c: int) -> None:
        if c == 1:
            out.append(np.sort(members))
            return
        node = pddp_node_split(Q, members, c, G, iters)
        split(node["left"], node["c_left"])
        split(node["right"], node["c_right"])

    if Nq == 0:
        return np.zeros(0, np.int64)
    split(np.arange(Nq, dtype=np.int64), -(-Nq // G))
    return np.concatenate(out)


def tree_nodes(Nq: int, G: int) -> List[Tuple[int, int, int, int]]:
    """Internal nodes of the PDDP tree as (level, start, size, n_groups).

    Because groups are emitted depth-first, every node is the contiguous range
    perm[start : start + size].  Shape depends only on (Nq, G).
    """
    nodes = []

    def walk(level, start, n, c):
        if c == 1:
            return
        nodes.append((level, start, n, c))
        nL = (c // 2) * G
        walk(level + 1, start, nL, c // 2)
        walk(level + 1, start + nL, n - nL, c - c // 2)

    if Nq > 0:
        walk(0, 0, Nq, -(-Nq // G))
    return nodes


def group_slices(Nq: int, G: int) -> List[slice]:
    return [slice(g * G, min((g + 1) * G, Nq)) for g in range(-(-Nq // G))]


# ---------------------------------------------------------------------------
# Exact per-group scores and token-level top-k selection
# ---------------------------------------------------------------------------
def column_mass(Q, K, lse: np.ndarray, members: np.ndarray, scale: float,
                causal_block: int = 0, q_offset: int = 0) -> np.ndarray:
    """Exact attention mass each key receives from a query group.

    m[j] = sum over i in the group of P_ij = exp(scale*<q_i,k_j> - lse_i),
    0 where j is not visible to i.  This is the group's exact attention score
    per KV token that the anchor step computes (MC-Sparse review, section 3).
    ``lse`` is the full-row log-normaliser of each member (indexed by original
    query index).
    """
    Q, K = _as64(Q), _as64(K)
    members = np.asarray(members, dtype=np.int64)
    logits = scale * (Q[members] @ K.T)
    vis = visible(members, np.arange(K.shape[0]), causal_block, q_offset)
    with np.errstate(invalid="ignore"):
        P = np.where(vis, np.exp(logits - lse[members][:, None]), 0.0)
    return P.sum(axis=0)


def topk_select(mass: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k keys with the largest mass, ties to the lower index,
    returned in ascending index order (token-level KV selection)."""
    mass = _as64(mass)
    order = np.lexsort((np.arange(mass.size), -mass))   # mass descending, index ascending
    return np.sort(order[:k])


# ---------------------------------------------------------------------------
# Residual-drift check (adaptive anchoring)
# ---------------------------------------------------------------------------
def sampled_drift(O, Q, K, V, rows, scale: float, causal_block: int = 0, q_offset: int = 0) -> float:
    """Relative distance of a step's output from exact attention on sampled
    query rows: ||O[rows] - O_exact[rows]||_F / ||O_exact[rows]||_F (0 when
    the exact rows are all zero).

    For a reuse output O = O_sparse + R_anchor, O - O_exact equals
    R_anchor - R_now, the movement of the dense-sparse residual since the
    anchor, measured against the output.  The review page (section 3) reuses
    selections and the residual because both are temporally stable; this is
    the quantity whose growth says that they no longer are, read here as the
    trigger for the next anchor.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    ex = np.zeros((rows.size, V.shape[1]), _F)
    for n, r in enumerate(rows):   # each sampled row at its own position q_offset + r
        ex[n] = dense_attention(Q[r:r + 1], K, V, scale, causal_block, q_offset + int(r))[0][0]
    ref = float(np.sqrt((ex ** 2).sum()))
    err = float(np.sqrt(((_as64(O)[rows] - ex) ** 2).sum()))
    return err / ref if ref > 0 else 0.0


# ---------------------------------------------------------------------------
# Block-sparse comparator: mean-pooled block selection
# ---------------------------------------------------------------------------
def block_scores(Q, K, rows: slice, scale: float, causal_block: int = 0, q_offset: int = 0,
                 block: int = 64) -> np.ndarray:
    """Mean-pooled score of every KV block for the query block ``rows``:
    scale*<mean of the query rows, mean of the block's key rows>, or -inf for
    a KV block none of whose keys is visible to any of the queries (see
    block_pooled_selection)."""
    Q, K = _as64(Q), _as64(K)
    Nkv = K.shape[0]
    qrows = np.arange(rows.start, rows.stop)
    qbar = Q[qrows].mean(axis=0)
    out = np.empty(-(-Nkv // block))
    for b in range(out.size):
        keys = np.arange(b * block, min((b + 1) * block, Nkv))
        seen = visible(qrows, keys, causal_block, q_offset).any()
        out[b] = scale * float(K[keys].mean(axis=0) @ qbar) if seen else -np.inf
    return out


def block_pooled_selection(Q, K, G: int, k: int, scale: float, causal_block: int = 0,
                           q_offset: int = 0, block: int = 64,
                           groups: Optional[Sequence[int]] = None) -> np.ndarray:
    """Selection of block-sparse attention with mean-pooled scoring, the
    approach MC-Sparse is measured against (review page, section 1 on
    selection error from approximate scoring such as mean pooling and on
    structural binding error; section 2 on block-granular sparsity).

    Readings (the page gives no formulas): query blocks are the G-token tiles
    of the token order and KV blocks the ``block``-token tiles (each last
    tile may be short); a block is represented by the mean of its rows, and
    the score of KV block b for query block g is scale*<mean q_g, mean k_b>.
    KV blocks none of whose keys is visible to any query of g rank after
    every other block.  Blocks are taken in order of decreasing score (ties to
    the lower block index) while the token count stays within k; the next
    block then contributes its lowest-index tokens up to exactly k.  Returns
    [c, k] token indices, ascending per row (rows of groups not listed in
    ``groups`` stay -1).
    """
    Q, K = _as64(Q), _as64(K)
    Nq, Nkv = Q.shape[0], K.shape[0]
    nkb = -(-Nkv // block)
    kb = [np.arange(b * block, min((b + 1) * block, Nkv)) for b in range(nkb)]
    sl = group_slices(Nq, G)
    out = np.full((len(sl), k), -1, dtype=np.int64)
    for g in (range(len(sl)) if groups is None else groups):
        score = block_scores(Q, K, sl[g], scale, causal_block, q_offset, block)
        order = np.lexsort((np.arange(nkb), -score))   # score descending, block index ascending
        sel: List[int] = []
        for b in order:
            sel.extend(kb[b][:k - len(sel)].tolist())
            if len(sel) == k:
                break
        out[g] = np.sort(np.asarray(sel, dtype=np.int64))
    return out


def block_sparse_step(Q, K, V, G: int, k: int, scale: float, causal_block: int = 0,
                      q_offset: int = 0, groups: Optional[Sequence[int]] = None):
    """One step of the block-sparse comparator: the mean-pooled selection of
    this step's Q/K, then attention of each query block over its selected
    tokens (no residual).  Query blocks are token-order tiles, so the grouping
    is the identity.  Returns (perm, idx, O)."""
    perm = np.arange(_as64(Q).shape[0], dtype=np.int64)
    idx = block_pooled_selection(Q, K, G, k, scale, causal_block, q_offset, groups=groups)
    O = sparse_attention(Q, K, V, perm, idx, G, scale, causal_block, q_offset, groups)
    return perm, idx, O


# ---------------------------------------------------------------------------
# Gathered sparse attention, residual and reuse
# ---------------------------------------------------------------------------
def sparse_attention(Q, K, V, perm: np.ndarray, idx: np.ndarray, G: int, scale: float,
                     causal_block: int = 0, q_offset: int = 0,
                     groups: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention of each group's queries over only that group's selected keys.

    For i in group g: O_i = sum over j in S_g visible to i of
    softmax_j(scale*<q_i,k_j>) v_j, the softmax renormalised over that
    selected visible set (a row with none gets 0).  Output rows are in the
    original token order; rows of groups not listed in ``groups`` stay 0.
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    perm = np.asarray(perm, dtype=np.int64)
    O = np.zeros((Q.shape[0], V.shape[1]), _F)
    sl = group_slices(Q.shape[0], G)
    for g in (range(len(sl)) if groups is None else groups):
        members = perm[sl[g]]
        sel = np.asarray(idx[g], dtype=np.int64)
        logits = scale * (Q[members] @ K[sel].T)
        vis = visible(members, sel, causal_block, q_offset)
        logits = np.where(vis, logits, -np.inf)
        mx = logits.max(axis=1)
        ok = np.isfinite(mx)
        E = np.exp(logits - np.where(ok, mx, 0.0)[:, None])
        den = E.sum(axis=1)
        P = np.where(ok[:, None], E / np.where(ok, den, 1.0)[:, None], 0.0)
        O[members] = P @ V[sel]
    return O


def anchor_step(Q, K, V, G: int, k: int, scale: float, causal_block: int = 0, q_offset: int = 0,
                iters: int = 32, perm: Optional[np.ndarray] = None):
    """Anchor step of MC-Sparse for one head (review page, section 3).

    Groups the queries (PDDP, unless ``perm`` is given), runs exact dense
    attention, ranks each group's KV tokens by exact attention mass and keeps
    the top k, runs sparse attention on that selection and stores the residual
    R = O_full - O_sparse.  Returns dict(perm, idx [c, k], O_full, lse, R).
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    if perm is None:
        perm = pddp_groups(Q, G, iters)
    O_full, lse = dense_attention(Q, K, V, scale, causal_block, q_offset)
    sl = group_slices(Q.shape[0], G)
    idx = np.stack([topk_select(column_mass(Q, K, lse, perm[s], scale, causal_block, q_offset), k)
                    for s in sl]) if sl else np.zeros((0, k), np.int64)
    O_sp = sparse_attention(Q, K, V, perm, idx, G, scale, causal_block, q_offset)
    return {"perm": perm, "idx": idx, "O_full": O_full, "lse": lse, "R": O_full - O_sp}


def reuse_step(Q, K, V, perm, idx, R, G: int, scale: float, causal_block: int = 0,
               q_offset: int = 0, groups: Optional[Sequence[int]] = None) -> np.ndarray:
    """Reuse step: sparse attention with the anchor's groups and selections on
    the current Q/K/V, plus the anchor's residual R as an additive correction."""
    O = sparse_attention(Q, K, V, perm, idx, G, scale, causal_block, q_offset, groups)
    return O + (_as64(R) if R is not None else 0.0)
