"""GPU checks of the residual-drift check (mcs_residual_drift) and of the
adaptive anchor schedule built on it.

MC-Sparse review, section 3: selections and the dense-sparse residual are
reused because they are temporally stable; the drift of a reuse output at
sampled rows is the residual's movement since the anchor, relative to the
output (oracle: sampled_drift).  Checked: identities that fix the value
(O = 0 gives 1; the library's own dense output gives its rounding only), the
drift of real reuse outputs against the oracle's on every head of the small
workloads and on sampled heads at full size, and the schedule's decisions.
"""

import numpy as np
import pytest

from oracle import mcs_oracle as orc
from sparse_attention_video_pddp_amd import synth
from tests.test_gpu_1_small_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def _drift(p, Q, K, V, O, rows):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    rows_t = torch.tensor(rows, dtype=torch.int32, device="cuda")
    drift = torch.full((p.B * p.H + 1,), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(mcs.workspace_size(p, mcs.MCS_WS_DRIFT)[0], 1), dtype=torch.uint8, device="cuda")
    mcs.residual_drift(p, Q, K, V, O, rows_t, drift, ws)
    torch.cuda.synchronize()
    d = drift.cpu().numpy()
    # the last value is the largest per-head drift, formed by the library
    assert d[-1] == d[:-1].max(), d
    return d[:-1].reshape(p.B, p.H)


def _tol(want):
    """Allowed |drift_gpu - drift_oracle|: the GPU's exact rows use bf16
    probabilities in the PV product (relative error ~2^-8 per row at most),
    so 5e-3 absolute plus 2% of the value."""
    return 5e-3 + 0.02 * want


@pytest.mark.parametrize("name", ["tiny", "bidir_small", "causal_small", "large_small", "stress_small"])
def test_drift_identities(cuda, name):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL[name]
    p = mcs.problem_for(w)
    (Q, K, V), _ = device_inputs(w, 0)
    rows = mcs.drift_rows(w.Nq, 64)
    zero = torch.zeros_like(Q)
    d0 = _drift(p, Q, K, V, zero, rows)
    assert np.all(np.abs(d0 - 1.0) < 1e-5), d0          # ||0 - X|| / ||X|| = 1
    Od = torch.empty_like(Q)
    mcs.dense_attn(p, Q, K, V, Od)
    dd = _drift(p, Q, K, V, Od, rows)
    assert np.all(dd >= 0) and np.all(dd < 1e-2), dd     # the dense output's own rounding


@pytest.mark.parametrize("name", list(SMALL))
def test_drift_of_reuse_output_matches_oracle(cuda, name):
    from sparse_attention_video_pddp_amd import mcs
    from tests.gpu_runner import log
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL[name]
    p = mcs.problem_for(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    (Q0, K0, V0), _ = device_inputs(w, 0)
    (Q1, K1, V1), host = device_inputs(w, 1, keep_heads=heads)
    st = mcs.MCSparseAttention(p)
    st.step(Q0, K0, V0, True)
    O = st.step(Q1, K1, V1, False)
    rows = mcs.drift_rows(w.Nq, 64)
    got = _drift(p, Q1, K1, V1, O, rows)
    for (b, h) in heads:
        q, k, v = (x.astype(np.float64) for x in host[(b, h)])
        Oh = O[b, h].float().cpu().numpy().astype(np.float64)
        want = orc.sampled_drift(Oh, q, k, v, rows, w.scale, w.causal_block, w.q_offset)
        tol = _tol(want)
        log(f"  {name} head {(b, h)}: drift {got[b, h]:.5f} oracle {want:.5f} (tol {tol:.1e})")
        assert abs(got[b, h] - want) <= tol


@pytest.mark.parametrize("name", ["bidir5", "causal", "large"])
def test_drift_full_size_sampled_heads(cuda, name):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    from tests.gpu_runner import log
    w = synth.get(name)
    p = mcs.problem_for(w)
    heads = [(0, 0), (0, w.H - 1)]
    (Q0, K0, V0), _ = device_inputs(w, 0, keep_heads=[])
    st = mcs.MCSparseAttention(p)
    st.step(Q0, K0, V0, True)
    del Q0, K0, V0
    (Q1, K1, V1), host = device_inputs(w, 1, keep_heads=heads)
    O = st.step(Q1, K1, V1, False)
    rows = mcs.drift_rows(w.Nq, 32)
    got = _drift(p, Q1, K1, V1, O, rows)
    torch.cuda.synchronize()
    for (b, h) in heads:
        q, k, v = (x.astype(np.float64) for x in host[(b, h)])
        Oh = O[b, h].float().cpu().numpy().astype(np.float64)
        want = orc.sampled_drift(Oh, q, k, v, rows, w.scale, w.causal_block, w.q_offset)
        tol = _tol(want)
        log(f"  {name} head {(b, h)}: drift {got[b, h]:.5f} oracle {want:.5f} (tol {tol:.1e})")
        assert abs(got[b, h] - want) <= tol


def test_adaptive_schedule_follows_the_drift(cuda):
    """A threshold between the drifts of consecutive reuse steps makes the
    schedule anchor exactly after the first step that crosses it, and every
    output equals the one a fixed schedule with the same anchors produces."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL["bidir_small"]
    p = mcs.problem_for(w)
    steps = [device_inputs(w, s)[0] for s in range(6)]
    # drifts of a fixed anchor-at-0 schedule decide the threshold
    probe = mcs.AdaptiveAnchoring(mcs.MCSparseAttention(p), threshold=float("inf"))
    for x in steps:
        probe.step(*x)
    d = [dr for a, dr in probe.history if not a]
    assert len(d) == 5 and all(np.isfinite(d)) and max(d) > min(d)
    thr = float(np.median(d))          # some reuse step crosses it
    ad = mcs.AdaptiveAnchoring(mcs.MCSparseAttention(p), threshold=thr)
    outs = [ad.step(*x).clone() for x in steps]
    anchors = [a for a, _ in ad.history]
    first_cross = next(i for i, (a, dr) in enumerate(ad.history) if not a and dr > thr)
    assert anchors[0] and anchors[first_cross + 1] and not any(anchors[1:first_cross + 1])
    ref = mcs.MCSparseAttention(p)
    for x, a, o in zip(steps, anchors, outs):
        assert torch.equal(ref.step(*x, a), o)
    # a period limit anchors without any drift crossing
    cap = mcs.AdaptiveAnchoring(mcs.MCSparseAttention(p), threshold=float("inf"), max_period=2)
    for x in steps:
        cap.step(*x)
    assert [a for a, _ in cap.history] == [True, False, True, False, True, False]


def test_adaptive_schedule_on_a_side_stream(cuda):
    """AdaptiveAnchoring handed a side stream without a stream context: the
    library's check runs on that stream and the binding reads the largest
    drift back on it too, so the drifts, anchor decisions and outputs equal
    those of the same schedule on the current stream bit for bit."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    w = SMALL["large_small"]
    p = mcs.problem_for(w)
    steps = [device_inputs(w, s)[0] for s in range(5)]
    torch.cuda.synchronize()

    def run(stream, threshold):
        ad = mcs.AdaptiveAnchoring(mcs.MCSparseAttention(p), threshold=threshold)
        outs = []
        for x in steps:
            O = ad.step(*x, stream=stream)
            (stream or torch.cuda.current_stream()).synchronize()
            outs.append(O.clone())
        return ad.history, outs

    hist0, _ = run(None, float("inf"))
    d = [dr for a, dr in hist0 if not a]
    assert len(d) == 4 and all(np.isfinite(d)) and max(d) > min(d)
    thr = float(np.median(d))
    ref_hist, ref_out = run(None, thr)
    side_hist, side_out = run(torch.cuda.Stream(), thr)
    assert side_hist == ref_hist and any(a for a, _ in ref_hist[1:])
    for a, b in zip(ref_out, side_out):
        assert torch.equal(a, b)
