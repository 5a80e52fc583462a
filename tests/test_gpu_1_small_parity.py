"""GPU parity at oracle-sized workloads (all heads, all groups, all rows).

Each workload is a scaled-down grid of one of the five benchmark workloads,
large enough to span several K/V tiles with a ragged tail, several PDDP
levels and a short last group.  The anchor runs on step 0, the reuse step on
step 1 (drifted inputs).  Every stage is compared with the fp64 oracle as
described in tests/parity.py.
"""
import numpy as np
import pytest

from sparse_attention_video_pddp_amd import synth
from tests.parity import assert_reports, check_head

pytestmark = pytest.mark.gpu

SMALL = {
    # fp32 smoke workload at its real size: 1024 tokens, G=64, k=103
    "tiny": synth.get("tiny"),
    # bidirectional, bf16: 720 tokens -> 12 groups (last 16), k=144 (3 tiles, last ragged)
    "bidir_small": synth.get("bidir5").with_(name="bidir_small", H=2, grid=(3, 12, 20), keep_permille=200),
    # frame-causal query chunk: 900 keys in frames of 150, queries = last 2 frames (300 -> 5 groups, last 44)
    "causal_small": synth.get("causal").with_(name="causal_small", H=2, grid=(6, 10, 15), q_frames=(4, 6),
                                              causal_block=150, keep_permille=100),
    # G=128, temperature 3/sqrt(d): 1200 tokens -> 10 groups (last 48), k=360
    "large_small": synth.get("large").with_(name="large_small", H=2, grid=(4, 15, 20), keep_permille=300),
    # 3D-local field generator, d=64, G=128: 2048 tokens -> 16 groups, k=205
    "stress_small": synth.get("stress").with_(name="stress_small", H=2, grid=(8, 16, 16), keep_permille=100),
    # query chunk in the middle of the video: the last two frames are visible to no query, so
    # their keys must get mass 0 (not whatever the workspace held) and never be selected
    "causal_mid": synth.get("causal").with_(name="causal_mid", H=2, grid=(6, 10, 15), q_frames=(2, 4),
                                            causal_block=150, keep_permille=100),
    # batch of two videos (B=2, H=2): every (b, h) has its own grouping, selection and residual
    "batch_small": synth.get("bidir5").with_(name="batch_small", B=2, H=2, grid=(2, 12, 20), keep_permille=150),
    # fp32 path with B=2
    "tiny_batch": synth.get("tiny").with_(name="tiny_batch", B=2, H=1, grid=(2, 16, 16)),
    # bf16, d=64 with groups of 64 (the stress workload has G=128): 960 tokens -> 15 groups, k=144
    "d64_g64": synth.get("bidir5").with_(name="d64_g64", H=2, d=64, grid=(4, 12, 20), keep_permille=150,
                                         scale=1.0 / 8.0),
    # queries sharing a mean far from the origin (30 x (1 + 0.5 z) per channel, ~40x the queries' own
    # spread): PDDP must centre each node without losing the spread.  4960 tokens, so the top
    # levels run the many-workgroup scatter kernels, the middle ones the one-workgroup node
    # kernel and the deep ones the small-node kernel; a mild logit scale keeps the attention
    # stages away from underflowing masses.  bf16, d=128, G=64 (78 groups, last 32), k=248
    "offset_d128_g64": synth.get("bidir5").with_(name="offset_d128_g64", H=2, grid=(8, 20, 31), keep_permille=50,
                                                 q_mean=30.0, scale=0.1 / 128 ** 0.5),
    # the same offset with d=64 and G=128: 2640 tokens (21 groups, last 80), k=264
    "offset_d64_g128": synth.get("bidir5").with_(name="offset_d64_g128", H=2, d=64, group_size=128,
                                                 grid=(6, 20, 22), keep_permille=100, q_mean=30.0,
                                                 scale=0.1 / 8.0),
    # fp32, d=128 with groups of 128, frame-causal: 900 queries of 1200 keys, k=120
    "f32_d128_g128": synth.get("tiny").with_(name="f32_d128_g128", H=2, d=128, group_size=128,
                                             grid=(8, 10, 15), q_frames=(2, 8), causal_block=150,
                                             keep_permille=100, scale=1.0 / 128 ** 0.5),
}


@pytest.fixture(scope="module")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_parity(cuda, name):
    from tests.gpu_runner import log, run_anchor_reuse
    w = SMALL[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cases = run_anchor_reuse(w, heads)
    for bh, case in cases.items():
        reps = check_head(case, w.group_size, w.k, w.scale, w.causal_block, w.q_offset, w.pddp_iters)
        for r in reps:
            log(f"  {name} head {bh}: {r}")
        assert_reports(reps, f"{name} head {bh}")


@pytest.mark.parametrize("name", ["bidir_small", "causal_small", "large_small", "stress_small", "d64_g64",
                                  "offset_d128_g64"])
def test_small_workload_parity_bf16_residual(cuda, name):
    """The same staged parity with the residual stored in bf16 (r_dtype
    MCS_BF16, one more rounding of R): every head, group and row."""
    from tests.gpu_runner import log, run_anchor_reuse
    w = SMALL[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cases = run_anchor_reuse(w, heads, r_dtype="bf16")
    for bh, case in cases.items():
        reps = check_head(case, w.group_size, w.k, w.scale, w.causal_block, w.q_offset, w.pddp_iters)
        for r in reps:
            log(f"  {name} (bf16 R) head {bh}: {r}")
        assert_reports(reps, f"{name} (bf16 R) head {bh}")


def test_dense_attn_matches_oracle_with_lse(cuda):
    import torch
    from oracle.mcs_oracle import dense_attention
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    for w in (SMALL["causal_small"], SMALL["stress_small"], SMALL["tiny"]):
        p = mcs.problem_for(w)
        (Q, K, V), host = device_inputs(w, 0, keep_heads=[(0, 1)])
        O = torch.empty_like(Q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        mcs.dense_attn(p, Q, K, V, O, lse)
        torch.cuda.synchronize()
        q, k, v = (x.astype(np.float64) for x in host[(0, 1)])
        Oo, lo = dense_attention(q, k, v, w.scale, w.causal_block, w.q_offset)
        vmax = np.abs(v).max()
        d = np.abs(O[0, 1].float().cpu().numpy() - Oo)
        assert d.max() <= 1e-2 * vmax and d.mean() <= 1e-3 * vmax, (w.name, d.max(), d.mean())
        dl = np.abs(lse[0, 1].cpu().numpy() - lo)
        assert dl.max() <= 1e-4 * max(1.0, np.abs(lo).max()), (w.name, dl.max())


def _state(w):
    from sparse_attention_video_pddp_amd import mcs
    return mcs.MCSparseAttention(mcs.problem_for(w))


def test_full_keep_sparse_equals_dense(cuda):
    """keep 100%: every group selects every key, so the GPU's sparse kernel
    (without R) must reproduce the GPU's dense kernel."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    for base in ("bidir_small", "causal_small"):
        w = SMALL[base].with_(keep_permille=1000)
        p = mcs.problem_for(w)
        (Q, K, V), _ = device_inputs(w, 0)
        st = _state(w)
        st.step(Q, K, V, True)
        assert torch.equal(st.idx[0, 0, 0], torch.arange(w.Nkv, dtype=torch.int32, device="cuda"))
        Od = torch.empty_like(Q)
        mcs.dense_attn(p, Q, K, V, Od)
        Os = torch.empty_like(Q)
        mcs.sparse_attn(p, Q, K, V, st.perm, st.idx, None, Os)
        torch.cuda.synchronize()
        vmax = V.float().abs().max().item()
        d = (Os.float() - Od.float()).abs()
        assert d.max().item() <= 1e-2 * vmax and d.mean().item() <= 1e-3 * vmax, (base, d.max().item())
        assert st.R.abs().max().item() <= 1e-2 * vmax


@pytest.mark.parametrize("name", ["bidir5", "causal", "large", "stress"])
def test_full_keep_at_full_length(cuda, name):
    """keep 100% at full length (k = Nkv kept keys per group, two heads:
    32760 keys for the benchmark's workload and the frame-causal chunk, 75600
    for large, 131072 for stress, whose mass rows are longer than the top-k
    kernel keeps in registers): every group selects every key, the sparse
    kernel without R reproduces the dense kernel and R vanishes to rounding.
    The frame-causal query chunk finds each query's visible prefix of a list
    far longer than the kernel's LDS scratch (its search runs in global
    memory)."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    from tests.gpu_runner import log
    w = synth.get(name).with_(H=2, keep_permille=1000)
    assert w.k == w.Nkv
    p = mcs.problem_for(w)
    (Q, K, V), _ = device_inputs(w, 0)
    st = _state(w)
    st.step(Q, K, V, True)
    full = torch.arange(w.Nkv, dtype=torch.int32, device="cuda")
    assert torch.equal(st.idx[0, 0, 0], full) and torch.equal(st.idx[0, 1, -1], full)
    Od = torch.empty_like(Q)
    mcs.dense_attn(p, Q, K, V, Od)
    Os = torch.empty_like(Q)
    mcs.sparse_attn(p, Q, K, V, st.perm, st.idx, None, Os)
    torch.cuda.synchronize()
    vmax = V.float().abs().max().item()
    d = (Os.float() - Od.float()).abs()
    log(f"  {name} keep 100%: max|sparse - dense| {d.max().item():.3e} mean {d.mean().item():.3e} "
        f"max|R| {st.R.abs().max().item():.3e} (vmax {vmax:.3f})")
    assert d.max().item() <= 1e-2 * vmax and d.mean().item() <= 1e-3 * vmax
    assert st.R.abs().max().item() <= 1e-2 * vmax


def test_zero_drift_reuse_returns_anchor_output(cuda):
    import torch
    from sparse_attention_video_pddp_amd.workload import device_inputs
    for base in ("bidir_small", "causal_small", "stress_small", "tiny"):
        w = SMALL[base]
        (Q, K, V), _ = device_inputs(w, 0)
        st = _state(w)
        Oa = st.step(Q, K, V, True).clone()
        Or = st.step(Q, K, V, False)
        torch.cuda.synchronize()
        vmax = V.float().abs().max().item()
        d = (Or.float() - Oa.float()).abs().max().item()
        assert d <= 1e-2 * vmax, (base, d)
        # R absorbs the discarded tail: reuse output equals the anchor's dense output to rounding
        assert d <= 2.0 ** -7 * max(1.0, Oa.float().abs().max().item()), (base, d)


def test_runs_are_bitwise_deterministic(cuda):
    import torch
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL["large_small"]
    (Q, K, V), _ = device_inputs(w, 0)
    outs = []
    for _ in range(2):
        st = _state(w)
        O = st.step(Q, K, V, True).clone()
        O2 = st.step(Q, K, V, False).clone()
        torch.cuda.synchronize()
        outs.append((st.perm.clone(), st.idx.clone(), st.R.clone(), O, O2))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_empty_query_set_is_a_noop(cuda):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    p = mcs.problem(1, 2, 0, 128, 64, 64, 10)
    x = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device="cuda")
    mcs.dense_attn(p, x, x, x, torch.empty_like(x))
    mcs.sparse_attn(p, x, x, x, torch.zeros(1, dtype=torch.int32, device="cuda"),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), None, torch.empty_like(x))
    torch.cuda.synchronize()


def test_single_group_and_single_key_edges(cuda):
    """Nq < G (one group, no PDDP split) and k = 1 (every query returns its
    group's one selected value row)."""
    import torch
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL["bidir_small"].with_(grid=(1, 5, 10), keep_permille=1)   # 50 tokens, k = 1
    assert w.k == 1 and w.n_groups == 1
    (Q, K, V), host = device_inputs(w, 0, keep_heads=[(0, 0)])
    st = _state(w)
    st.step(Q, K, V, True)
    Os = st.step(Q, K, V, False)
    torch.cuda.synchronize()
    assert torch.equal(st.perm[0, 0], torch.arange(50, dtype=torch.int32, device="cuda"))
    j = int(st.idx[0, 0, 0, 0])
    # sparse part of every row is V[j]; reuse O = V[j] + R = O_full (to rounding)
    R = st.R[0, 0]
    sp = (Os[0, 0].float() - R)
    assert (sp - V[0, 0, j].float()).abs().max().item() <= 2e-2


def test_side_stream_gives_the_default_stream_results(cuda):
    """Every entry point enqueues on the stream it is given: the whole anchor
    + reuse sequence on a side stream (default priority) matches the same
    sequence on the default stream bit for bit, and waiting on that stream
    alone makes the results visible."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL["bidir_small"]
    p = mcs.problem_for(w)
    (Q, K, V), _ = device_inputs(w, 0)
    (Q1, K1, V1), _ = device_inputs(w, 1)

    def run(stream):
        st = mcs.MCSparseAttention(p)
        with torch.cuda.stream(stream):
            O0 = st.step(Q, K, V, True, stream=stream).clone()
            O1 = st.step(Q1, K1, V1, False, stream=stream).clone()
            Od = torch.empty_like(Q)
            mcs.dense_attn(p, Q1, K1, V1, Od, stream=stream)
        stream.synchronize()
        return st.perm, st.idx, st.R, O0, O1, Od

    torch.cuda.synchronize()
    ref = run(torch.cuda.current_stream())
    side = run(torch.cuda.Stream())
    for a, b in zip(ref, side):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["bidir_small", "causal_small", "causal_mid", "large_small", "stress_small",
                                  "d64_g64", "offset_d128_g64", "batch_small"])
def test_single_pass_anchor_equals_two_pass(cuda, name):
    """The single-pass anchor (each group's column mass kept on chip and
    selected in the same workgroup) computes every mass with the two-pass
    path's arithmetic: the selections, and therefore the residual and the
    anchor and reuse outputs, are equal bit for bit; the single pass is also
    checked against the oracle stage by stage."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    from tests.gpu_runner import log, run_anchor_reuse
    w = SMALL[name]
    (Q0, K0, V0), _ = device_inputs(w, 0)
    (Q1, K1, V1), _ = device_inputs(w, 1)
    res = {}
    for mode in ("two_pass", "single_pass"):
        st = mcs.MCSparseAttention(mcs.problem_for(w, anchor_mode=mode))
        Oa = st.step(Q0, K0, V0, True).clone()
        Or = st.step(Q1, K1, V1, False).clone()
        torch.cuda.synchronize()
        res[mode] = (st.perm.clone(), st.idx.clone(), st.R.clone(), Oa, Or)
    for a, b in zip(res["two_pass"], res["single_pass"]):
        assert torch.equal(a, b)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    cases = run_anchor_reuse(w, heads, anchor_mode="single_pass")
    for bh, case in cases.items():
        reps = check_head(case, w.group_size, w.k, w.scale, w.causal_block, w.q_offset, w.pddp_iters)
        for r in reps:
            log(f"  {name} (single pass) head {bh}: {r}")
        assert_reports(reps, f"{name} (single pass) head {bh}")


@pytest.mark.parametrize("chunk", [0, 3, 6])
def test_single_pass_anchor_at_full_size(cuda, chunk):
    """Chunks of the frame-causal video at full size (4680 queries over a
    32760-row K/V cache, 12 heads; chunk c sees 4680 (c + 1) keys, up to the
    single pass's largest row): both anchor modes give the same selections."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    base = synth.get("causal")
    w = base.with_(name=f"causal_chunk{chunk}", q_frames=(3 * chunk, 3 * chunk + 3))
    (Q, K, V), _ = device_inputs(w, 0)
    idx = {}
    for mode in ("two_pass", "single_pass"):
        st = mcs.MCSparseAttention(mcs.problem_for(w, anchor_mode=mode))
        st.step(Q, K, V, True)
        torch.cuda.synchronize()
        idx[mode] = st.idx.clone()
    assert torch.equal(idx["two_pass"], idx["single_pass"])
