"""GPU parity of the block-sparse comparator (mcs_block_select followed by
mcs_sparse_attn without a residual) against the fp64 oracle.

MC-Sparse review, sections 1-2: block-sparse attention with mean-pooled block
scores, the selection recomputed on every step.  At the oracle-sized
workloads every head and every query block is checked: the identity grouping
bit for bit, each token list against the oracle's (near-ties of the pooled
scores validated as described in tests/parity.py) and the output against the
oracle's attention over the GPU's lists.  At full size, sampled query blocks
of three workloads are checked the same way.
"""
import numpy as np
import pytest

from oracle import mcs_oracle as orc
from sparse_attention_video_pddp_amd import synth
from tests.parity import MAX_TOL, MEAN_TOL, check_block_selection
from tests.test_gpu_1_small_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def _run(w, step, heads):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    from tests.gpu_runner import log
    p = mcs.problem_for(w)
    log(f"[gpu] block-sparse {w.name}: {p}")
    (Q, K, V), host = device_inputs(w, step, keep_heads=heads)
    cmp_ = mcs.BlockSparseComparator(p)
    O = cmp_.step(Q, K, V)
    torch.cuda.synchronize()
    return cmp_, O, host, (Q, K, V)


def _check_head(w, cmp_, O, host, b, h, groups):
    q, k, v = (x.astype(np.float64) for x in host[(b, h)])
    perm = cmp_.perm[b, h].cpu().numpy()
    assert np.array_equal(perm, np.arange(w.Nq)), "grouping is not the identity"
    idx = cmp_.idx[b, h].cpu().numpy().astype(np.int64)
    for g in groups:
        err = check_block_selection(q, k, idx[g], g, w.group_size, w.k, w.scale, w.causal_block, w.q_offset)
        assert err is None, f"{w.name} head {(b, h)}: {err}"
    ref = orc.sparse_attention(q, k, v, perm, idx, w.group_size, w.scale, w.causal_block, w.q_offset,
                               groups=groups)
    rows = np.concatenate([np.arange(w.Nq)[s] for s in (orc.group_slices(w.Nq, w.group_size)[g] for g in groups)])
    got = O[b, h].float().cpu().numpy().astype(np.float64)[rows]
    d = np.abs(got - ref[rows])
    vmax = np.abs(v).max()
    assert np.all(np.isfinite(got))
    assert d.max() <= MAX_TOL * vmax and d.mean() <= MEAN_TOL * vmax, (w.name, (b, h), d.max(), d.mean())
    return d.max(), d.mean()


@pytest.mark.parametrize("name", list(SMALL))
def test_block_sparse_small_parity(cuda, name):
    from tests.gpu_runner import log
    w = SMALL[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cmp_, O, host, _ = _run(w, 1, heads)
    for (b, h) in heads:
        mx, mn = _check_head(w, cmp_, O, host, b, h, range(w.n_groups))
        log(f"  {name} head {(b, h)}: {w.n_groups} blocks ok, O max|d|={mx:.3e} mean|d|={mn:.3e}")


def test_block_sparse_full_budget_equals_dense(cuda):
    """k = Nkv: every query block keeps every token, so the comparator's output
    is the library's dense attention."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    for base in ("bidir_small", "causal_small", "tiny"):
        w = SMALL[base].with_(keep_permille=1000)
        cmp_, O, _, (Q, K, V) = _run(w, 0, [])
        Od = torch.empty_like(Q)
        mcs.dense_attn(mcs.problem_for(w), Q, K, V, Od)
        torch.cuda.synchronize()
        assert torch.equal(cmp_.idx[0, 0, 0], torch.arange(w.Nkv, dtype=torch.int32, device="cuda"))
        vmax = V.float().abs().max().item()
        d = (O.float() - Od.float()).abs()
        assert d.max().item() <= MAX_TOL * vmax and d.mean().item() <= MEAN_TOL * vmax, (base, d.max().item())


@pytest.mark.parametrize("name", ["bidir5", "causal", "stress"])
def test_block_sparse_full_size_sampled(cuda, name):
    from tests.gpu_runner import log
    w = synth.get(name)
    heads = [(0, 0), (0, w.H - 1)]
    cmp_, O, host, _ = _run(w, 1, heads)
    rng = np.random.default_rng(7)
    groups = sorted({0, w.n_groups - 1, *rng.choice(w.n_groups, 4, replace=False).tolist()})
    for (b, h) in heads:
        mx, mn = _check_head(w, cmp_, O, host, b, h, groups)
        log(f"  {name} head {(b, h)} blocks {groups}: ok, O max|d|={mx:.3e} mean|d|={mn:.3e}")


LONG = {
    # 196608 keys -> 3072 KV blocks: the sort path at its largest padding (4096 pairs)
    "long_kv_sort": synth.get("stress").with_(name="long_kv_sort", H=1, grid=(48, 64, 64)),
    # 270336 keys -> 4224 KV blocks: beyond the sort path, the radix block select
    "long_kv_radix": synth.get("stress").with_(name="long_kv_radix", H=1, grid=(66, 64, 64)),
}


@pytest.mark.parametrize("name", list(LONG))
def test_block_sparse_long_kv_sampled(cuda, name):
    from tests.gpu_runner import log
    w = LONG[name]
    cmp_, O, host, _ = _run(w, 1, [(0, 0)])
    rng = np.random.default_rng(11)
    groups = sorted({0, w.n_groups - 1, *rng.choice(w.n_groups, 3, replace=False).tolist()})
    mx, mn = _check_head(w, cmp_, O, host, 0, 0, groups)
    log(f"  {name} ({-(-w.Nkv // 64)} KV blocks) blocks {groups}: ok, O max|d|={mx:.3e} mean|d|={mn:.3e}")
