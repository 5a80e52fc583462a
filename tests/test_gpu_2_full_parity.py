"""GPU parity at the full benchmark sizes, on sampled outputs.

The five workloads run at their real shapes through the same entry points the
benchmark times (mcs_group + mcs_anchor on step 0, mcs_sparse_attn on step 1).
For two sampled heads of each, the oracle recomputes the whole PDDP grouping
of the head, the top-k selection, residual and reuse output of sampled groups
(always including the short last group) and the exact attention of sampled
rows; see tests/parity.py for the stage rules and tolerances.
"""
import numpy as np
import pytest

from sparse_attention_video_pddp_amd import synth
from tests.parity import assert_reports, check_head

pytestmark = pytest.mark.gpu

FULL = ["causal", "bidir5", "bidir10", "large", "stress"]


def sample_groups(c: int, rng, n: int = 4):
    pick = {0, c - 1, c // 2}
    while len(pick) < min(c, n + 3):
        pick.add(int(rng.integers(0, c)))
    return sorted(pick)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    import torch
    from tests.gpu_runner import log, run_anchor_reuse
    assert torch.cuda.is_available()
    w = synth.get(name)
    heads = [(0, 0), (0, w.H - 1)]
    cases = run_anchor_reuse(w, heads)
    rng = np.random.default_rng(w.cfg_id * 100 + w.keep_permille)
    for bh, case in cases.items():
        groups = sample_groups(w.n_groups, rng)
        rows = np.unique(np.concatenate([[0, w.Nq - 1], rng.integers(0, w.Nq, 254)]))
        reps = check_head(case, w.group_size, w.k, w.scale, w.causal_block, w.q_offset, w.pddp_iters,
                          groups=groups, rows=rows)
        for r in reps:
            log(f"  {name} head {bh} groups {groups}: {r}")
        assert_reports(reps, f"{name} head {bh}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["bidir5", "causal", "large", "stress"])
def test_full_size_groups_every_head(name):
    """mcs_group at the full size, every head: each split recomputed by the
    oracle from the GPU's parent set (check_groups_nodewise); the many-
    workgroup levels derive a right child's sums from its parent's and its
    sibling's, so every head's top levels are covered here.  (bidir10's
    queries are bidir5's: the keep fraction does not enter the grouping.)"""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    from tests.gpu_runner import log
    from tests.parity import check_groups_nodewise
    assert torch.cuda.is_available()
    w = synth.get(name)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    p = mcs.problem_for(w)
    (Q, K, V), host = device_inputs(w, 0, keep_heads=heads)
    del K, V
    perm = torch.empty((w.B, w.H, w.Nq), dtype=torch.int32, device=Q.device)
    g, _ = mcs.workspace_size(p, mcs.MCS_WS_GROUP)
    ws = torch.empty(max(g, 1), dtype=torch.uint8, device=Q.device)
    mcs.group(p, Q, perm, ws)
    torch.cuda.synchronize()
    perm_h = perm.cpu().numpy()
    for (b, h) in heads:
        rep = check_groups_nodewise(host[(b, h)][0].astype(np.float64), perm_h[b, h], w.group_size, w.pddp_iters)
        log(f"  {name} head {(b, h)}: {rep}")
        assert rep.ok, f"{name} head {(b, h)}: {rep}"
