"""GPU parity of attention over a foreign K/V cache (cross-inference cache
attention, CHAI summary, section B: the current generation's queries attend
to the keys and values cached from an earlier generation).

Computationally this is the library's attention with keys and values from
another source and Nq != Nkv, no mask: the dense kernel, and the whole
anchor/reuse path with the cache held fixed while the queries drift.  Inputs:
queries from the bidirectional workload's generator on a 3 x 12 x 20 grid,
the cache from the same generator with another seed namespace on a
4 x 12 x 20 grid (960 cached tokens, 720 queries).  Checked like the other
workloads (tests/parity.py) on every head.
"""
import numpy as np
import pytest

from oracle import mcs_oracle as orc
from sparse_attention_video_pddp_amd import synth
from tests.parity import HeadCase, MAX_TOL, MEAN_TOL, assert_reports, check_head

pytestmark = pytest.mark.gpu

WQ = synth.get("bidir5").with_(name="cache_q", H=2, grid=(3, 12, 20), keep_permille=150)
WKV = WQ.with_(name="cache_kv", cfg_id=97, grid=(4, 12, 20))


@pytest.fixture(scope="module")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def test_attention_over_a_foreign_cache(cuda):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import _to_tensor
    from tests.gpu_runner import log
    k = (WKV.Nkv * WQ.keep_permille + 999) // 1000
    p = mcs.problem(WQ.B, WQ.H, WQ.Nq, WKV.Nkv, WQ.d, WQ.group_size, k, WQ.scale, dtype=WQ.dtype,
                    pddp_iters=WQ.pddp_iters)
    q0, q1, kv = [], [], []
    for h in range(WQ.H):
        q0.append(synth.head_inputs(WQ, 0, h, 0)[0])
        q1.append(synth.head_inputs(WQ, 0, h, 1)[0])
        _, kk, vv = synth.head_inputs(WKV, 0, h, 0)
        kv.append((kk, vv))
    dev = lambda xs: torch.stack([_to_tensor(x, WQ.dtype) for x in xs])[None].to("cuda")  # noqa: E731
    Q0, Q1 = dev(q0), dev(q1)
    K, V = dev([a for a, _ in kv]), dev([b for _, b in kv])
    # dense attention over the cache, with lse
    Od = torch.empty_like(Q0)
    lse = torch.empty((1, WQ.H, WQ.Nq), dtype=torch.float32, device="cuda")
    mcs.dense_attn(p, Q0, K, V, Od, lse)
    st = mcs.MCSparseAttention(p)
    O0 = st.step(Q0, K, V, True).clone()
    O1 = st.step(Q1, K, V, False).clone()
    torch.cuda.synchronize()
    for h in range(WQ.H):
        f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
        kk, vv = f64(kv[h][0]), f64(kv[h][1])
        ref, lref = orc.dense_attention(f64(q0[h]), kk, vv, WQ.scale)
        vmax = np.abs(vv).max()
        d = np.abs(Od[0, h].float().cpu().numpy() - ref)
        assert d.max() <= MAX_TOL * vmax and d.mean() <= MEAN_TOL * vmax, (h, d.max(), d.mean())
        assert np.abs(lse[0, h].cpu().numpy() - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max())
        case = HeadCase(f64(q0[h]), kk, vv, f64(q1[h]), kk, vv,
                        perm=st.perm[0, h].cpu().numpy(), idx=st.idx[0, h].cpu().numpy(),
                        O_full=O0[0, h].float().cpu().numpy().astype(np.float64),
                        R=st.R[0, h].float().cpu().numpy().astype(np.float64),
                        O_reuse=O1[0, h].float().cpu().numpy().astype(np.float64))
        reps = check_head(case, WQ.group_size, k, WQ.scale, 0, 0, WQ.pddp_iters)
        for r in reps:
            log(f"  cache attention head {h}: {r}")
        assert_reports(reps, f"cache attention head {h}")


def _foreign_cache_case(kv_grid, k, cfg_id, label):
    """128 queries (two groups) over a one-head cache of the given grid, k
    kept keys per group: anchor and reuse on the GPU, every stage checked
    against the oracle."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import _to_tensor
    from tests.gpu_runner import log
    wq = WQ.with_(name="one_head_q", H=1, grid=(1, 8, 16))
    wkv = wq.with_(name="one_head_kv", cfg_id=cfg_id, grid=kv_grid)
    assert wq.Nq == 128
    p = mcs.problem(1, 1, wq.Nq, wkv.Nkv, wq.d, wq.group_size, k, wq.scale, dtype=wq.dtype,
                    pddp_iters=wq.pddp_iters)
    q0 = synth.head_inputs(wq, 0, 0, 0)[0]
    q1 = synth.head_inputs(wq, 0, 0, 1)[0]
    _, kk, vv = synth.head_inputs(wkv, 0, 0, 0)
    dev = lambda x: _to_tensor(x, wq.dtype)[None, None].to("cuda")  # noqa: E731
    Q0, Q1, K, V = dev(q0), dev(q1), dev(kk), dev(vv)
    st = mcs.MCSparseAttention(p)
    O0 = st.step(Q0, K, V, True).clone()
    O1 = st.step(Q1, K, V, False).clone()
    torch.cuda.synchronize()
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    kd, vd = f64(kk), f64(vv)
    case = HeadCase(f64(q0), kd, vd, f64(q1), kd, vd,
                    perm=st.perm[0, 0].cpu().numpy(), idx=st.idx[0, 0].cpu().numpy(),
                    O_full=O0[0, 0].float().cpu().numpy().astype(np.float64),
                    R=st.R[0, 0].float().cpu().numpy().astype(np.float64),
                    O_reuse=O1[0, 0].float().cpu().numpy().astype(np.float64))
    reps = check_head(case, wq.group_size, k, wq.scale, 0, 0, wq.pddp_iters)
    for r in reps:
        log(f"  {label}: {r}")
    assert_reports(reps, label)


def test_large_kept_key_count(cuda):
    """A large selection: k = 28672 kept keys per group out of a 30240-key
    cache (472.5 key tiles: a ragged tail; the gathered kernel streams the
    offsets of 896 tiles through its eight-tile ring), two groups of 64
    queries.  The boundary of the top-k then lies deep in the low-mass tail,
    where near-ties are common; tests/parity.py validates the GPU's choice
    there."""
    _foreign_cache_case((12, 40, 63), 28672, 98, "k = 28672 of 30240 keys")


def test_top_k_over_rows_longer_than_the_register_cache(cuda):
    """Mass rows of 100000 keys: more than the top-k kernel keeps in
    registers (81920), so its block select re-reads the row from memory on
    every pass (sixteen keys per thread in flight); every group is checked."""
    _foreign_cache_case((25, 40, 100), 2000, 99, "k = 2000 of 100000 keys")
