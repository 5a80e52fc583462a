"""Staged parity checks of GPU results against the fp64 oracle.

The oracle runs end to end on its own results (its own PDDP grouping, its own
top-k selections).  fp32 on the GPU and fp64 in the oracle may legitimately
decide a near-tie differently; only then is the GPU's choice validated
instead of compared, and the later stages of that group are computed on the
validated choice, so one near-tie cannot cascade:
  * groups: perm must equal the oracle's grouping, or else be a valid grouping
    whose every split equals the oracle's split of the GPU's parent set except
    tokens whose oracle projection lies within 1e-5 * max|p| of the split point;
  * top-k: each group's selection must equal the oracle's, or else differ
    only in keys whose oracle mass is within 1e-5 relative of the k-th mass;
  * block-sparse comparator: each query block's token list must equal the
    oracle's, or else be whole blocks plus one partial block (its lowest
    tokens) differing from the oracle's only in blocks whose oracle score lies
    within 1e-5 * max|score| of the score of the oracle's last block taken;
  * outputs (O_full, R, reuse O): max|dO| <= 1e-2 * max|V| and
    mean|dO| <= 1e-3 * max|V| (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

from oracle import mcs_oracle as orc

SPLIT_BAND = 1e-5
TOPK_BAND = 1e-5
MAX_TOL = 1e-2
MEAN_TOL = 1e-3


@dataclasses.dataclass
class StageReport:
    name: str
    ok: bool
    detail: str

    def __str__(self):
        return f"[{'ok' if self.ok else 'FAIL'}] {self.name}: {self.detail}"


def check_perm_structure(perm: np.ndarray, Nq: int, G: int) -> StageReport:
    perm = np.asarray(perm, dtype=np.int64)
    if perm.shape != (Nq,) or not np.array_equal(np.sort(perm), np.arange(Nq)):
        return StageReport("perm structure", False, "not a permutation of [0, Nq)")
    for s in orc.group_slices(Nq, G):
        if np.any(np.diff(perm[s]) <= 0):
            return StageReport("perm structure", False, f"group {s.start // G} members not ascending")
    return StageReport("perm structure", True, f"{-(-Nq // G)} groups")


def check_groups_nodewise(Q: np.ndarray, perm: np.ndarray, G: int, iters: int,
                          max_nodes: Optional[int] = None) -> StageReport:
    """Recompute every split (or the first ``max_nodes`` in level order) from
    the GPU's parent set and compare the GPU's left child with the oracle's."""
    st = check_perm_structure(perm, Q.shape[0], G)
    if not st.ok:
        return st
    perm = np.asarray(perm, dtype=np.int64)
    nodes = sorted(orc.tree_nodes(Q.shape[0], G))
    if max_nodes is not None:
        nodes = nodes[:max_nodes]
    exempt = 0
    for level, start, size, c in nodes:
        members = np.sort(perm[start:start + size])
        node = orc.pddp_node_split(Q, members, c, G, iters)
        nL = node["c_left"] * G
        gpu_left = set(perm[start:start + nL].tolist())
        ora_left = set(node["left"].tolist())
        diff = gpu_left.symmetric_difference(ora_left)
        if not diff:
            continue
        p = node["p"]
        pos = {int(m): i for i, m in enumerate(members)}
        band = SPLIT_BAND * np.abs(p).max()
        gaps = [abs(p[pos[t]] - node["split_point"]) for t in diff]
        if max(gaps) > band:
            return StageReport("groups", False,
                               f"level {level} node@{start} (n={size}): {len(diff)} tokens on the wrong side, "
                               f"max gap to split {max(gaps):.3e} > band {band:.3e}")
        exempt += len(diff)
    return StageReport("groups", True, f"{len(nodes)} splits checked, {exempt} near-tie tokens exempt")


def check_topk(mass_oracle: np.ndarray, idx_gpu: np.ndarray, k: int, group: int) -> Optional[str]:
    """None if the GPU's selection equals the oracle's up to near-ties."""
    sel = np.asarray(idx_gpu, dtype=np.int64)
    if sel.shape != (k,) or np.any(np.diff(sel) <= 0) or sel.min() < 0 or sel.max() >= mass_oracle.size:
        return f"group {group}: selection is not {k} unique ascending in-range indices"
    ora = orc.topk_select(mass_oracle, k)
    diff = np.setxor1d(sel, ora)
    if diff.size == 0:
        return None
    mk = np.sort(mass_oracle)[::-1][k - 1]
    gap = np.abs(mass_oracle[diff] - mk)
    if np.all(gap <= TOPK_BAND * mk):
        return None
    return (f"group {group}: {diff.size} keys differ, max |m - m_k| = {gap.max():.3e} "
            f"> {TOPK_BAND} * m_k = {TOPK_BAND * mk:.3e}")


def check_block_selection(Q: np.ndarray, K: np.ndarray, idx_gpu: np.ndarray, g: int, G: int, k: int,
                          scale: float, causal_block: int, q_offset: int, block: int = 64) -> Optional[str]:
    """None if the GPU's block-sparse selection of query block g equals the
    oracle's up to near-ties of the pooled block scores."""
    Nq, Nkv = Q.shape[0], K.shape[0]
    sel = np.asarray(idx_gpu, dtype=np.int64)
    if sel.shape != (k,) or np.any(np.diff(sel) <= 0) or sel.min() < 0 or sel.max() >= Nkv:
        return f"block {g}: selection is not {k} unique ascending in-range indices"
    ora = orc.block_pooled_selection(Q, K, G, k, scale, causal_block, q_offset, block, groups=[g])[g]
    if np.array_equal(sel, ora):
        return None
    nkb = -(-Nkv // block)
    size = np.minimum(block, Nkv - block * np.arange(nkb))
    got = np.bincount(sel // block, minlength=nkb)
    want = np.bincount(ora // block, minlength=nkb)
    part = np.flatnonzero((got > 0) & (got < size))
    if part.size > 1 or any(sel[sel // block == b].tolist() != list(range(b * block, b * block + got[b]))
                            for b in part):
        return f"block {g}: selection is not whole blocks plus the lowest tokens of one block"
    score = orc.block_scores(Q, K, orc.group_slices(Nq, G)[g], scale, causal_block, q_offset, block)
    finite = score[np.isfinite(score)]
    band = TOPK_BAND * (np.abs(finite).max() if finite.size else 1.0)
    order = np.lexsort((np.arange(nkb), -score))
    last = order[np.flatnonzero(want[order] > 0).max()]          # the oracle's last block taken
    differ = np.flatnonzero(got != want)
    gap = np.abs(score[differ] - score[last])
    if np.all(np.isfinite(score[differ])) and np.isfinite(score[last]) and np.all(gap <= band):
        return None
    return (f"block {g}: {differ.size} KV blocks taken differently, max score gap to the boundary "
            f"{np.nanmax(gap) if gap.size else 0.0:.3e} > band {band:.3e}")


def compare(name: str, got: np.ndarray, ref: np.ndarray, vmax: float) -> StageReport:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    mx, mn = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    ok = mx <= MAX_TOL * vmax and mn <= MEAN_TOL * vmax and np.all(np.isfinite(got))
    return StageReport(name, bool(ok), f"max|d|={mx:.3e} (tol {MAX_TOL * vmax:.3e}) "
                                       f"mean|d|={mn:.3e} (tol {MEAN_TOL * vmax:.3e})")


@dataclasses.dataclass
class HeadCase:
    """One head's anchor and reuse inputs (float64 copies of the exact values
    the GPU consumed) and the GPU's outputs for it."""
    Q0: np.ndarray
    K0: np.ndarray
    V0: np.ndarray
    Q1: np.ndarray
    K1: np.ndarray
    V1: np.ndarray
    perm: np.ndarray
    idx: np.ndarray
    O_full: np.ndarray
    R: np.ndarray
    O_reuse: np.ndarray


def check_head(case: HeadCase, G: int, k: int, scale: float, causal_block: int, q_offset: int, iters: int,
               groups: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
               max_nodes: Optional[int] = None) -> List[StageReport]:
    """Staged parity of one head.  ``groups``/``rows`` restrict the checks to
    sampled groups and dense rows (full-size workloads); None = all.

    The oracle runs on its own results: its own PDDP grouping and its own
    top-k selections.  Only where the GPU's result legitimately differs (a
    split or selection decided by a near-tie, see the module docstring) is the
    GPU's choice validated instead, and the later stages of that group are then
    computed on the validated choice; the reports count such cases.
    """
    reps = []
    Nq = case.Q0.shape[0]
    sl = orc.group_slices(Nq, G)
    gsel = list(range(len(sl))) if groups is None else list(groups)
    perm_gpu = np.asarray(case.perm, np.int64)
    perm_o = orc.pddp_groups(case.Q0, G, iters)
    if np.array_equal(perm_o, perm_gpu):
        reps.append(StageReport("groups", True, "bit-exact with the oracle's PDDP grouping"))
        perm_ref = perm_o
    else:
        r = check_groups_nodewise(case.Q0, perm_gpu, G, iters, max_nodes)
        reps.append(StageReport("groups", r.ok, "differs from the oracle's grouping; validated split by "
                                                "split: " + r.detail))
        perm_ref = perm_gpu
    # dense rows (anchor inputs)
    drows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    Od, _ = orc.dense_attention(case.Q0, case.K0, case.V0, scale, causal_block, q_offset, rows=drows)
    vmax0 = float(np.abs(case.V0).max())
    reps.append(compare("O_full (dense rows)", case.O_full[drows], Od, vmax0))
    # top-k: the oracle's own selection per group
    msgs, exact, band = [], 0, 0
    idx_ref = np.zeros((len(sl), k), np.int64)
    member_rows = np.concatenate([perm_ref[sl[g]] for g in gsel])
    Ofull_m, lse_m = orc.dense_attention(case.Q0, case.K0, case.V0, scale, causal_block, q_offset,
                                         rows=member_rows)
    lse_full = np.full(Nq, np.nan)
    lse_full[member_rows] = lse_m
    for g in gsel:
        members = perm_ref[sl[g]]
        m = orc.column_mass(case.Q0, case.K0, lse_full, members, scale, causal_block, q_offset)
        own = orc.topk_select(m, k)
        if np.array_equal(own, np.asarray(case.idx[g], np.int64)):
            exact += 1
            idx_ref[g] = own
            continue
        e = check_topk(m, case.idx[g], k, g)
        if e:
            msgs.append(e)
        else:
            band += 1
            idx_ref[g] = np.asarray(case.idx[g], np.int64)
    reps.append(StageReport("top-k", not msgs, msgs[0] if msgs else
                            f"{exact} groups bit-exact, {band} equal up to near-ties"))
    # residual and reuse on the reference groups and selections
    Osp0 = orc.sparse_attention(case.Q0, case.K0, case.V0, perm_ref, idx_ref, G, scale, causal_block, q_offset,
                                groups=gsel)[member_rows]
    R_ora = Ofull_m - Osp0
    reps.append(compare("R (anchor residual)", case.R[member_rows], R_ora, vmax0))
    Osp1 = orc.sparse_attention(case.Q1, case.K1, case.V1, perm_ref, idx_ref, G, scale, causal_block, q_offset,
                                groups=gsel)[member_rows]
    reps.append(compare("O (reuse step)", case.O_reuse[member_rows], Osp1 + R_ora,
                        float(np.abs(case.V1).max())))
    return reps


def assert_reports(reps: Iterable[StageReport], context: str = "") -> None:
    reps = list(reps)
    bad = [r for r in reps if not r.ok]
    if bad:
        raise AssertionError(context + "\n" + "\n".join(str(r) for r in reps))
