"""The allocation-free drift check (mcs_residual_drift_noalloc) against the
workspace entry point (mcs_residual_drift): two calls in a row through the C
ABI, the second on a smaller problem with fewer sampled rows, each equal to
the workspace entry point's result on the same inputs bit for bit (the same
kernels on the same data layout); a problem whose scratch exceeds the static
array is refused on the host."""
import numpy as np
import pytest

from sparse_attention_video_pddp_amd import synth

pytestmark = pytest.mark.gpu


def _case(w, n_rows, r_dtype="f32"):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import device_inputs
    p = mcs.problem_for(w, r_dtype)
    (Q0, K0, V0), _ = device_inputs(w, 0)
    (Q1, K1, V1), _ = device_inputs(w, 1)
    st = mcs.MCSparseAttention(p)
    st.step(Q0, K0, V0, True)
    O = st.step(Q1, K1, V1, False)
    rows = torch.tensor(mcs.drift_rows(w.Nq, n_rows), dtype=torch.int32, device="cuda")
    return p, (Q1, K1, V1, O, rows)


def test_noalloc_drift_equals_workspace_drift():
    import torch
    from sparse_attention_video_pddp_amd import mcs
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    # first call: 12 groups x 2 heads, 128 rows; second: a smaller video, fewer heads and rows
    big = synth.get("bidir5").with_(name="noalloc_big", H=3, grid=(3, 12, 20), keep_permille=200)
    small = synth.get("causal").with_(name="noalloc_small", H=1, grid=(4, 8, 10), q_frames=(2, 4),
                                      causal_block=80, keep_permille=150)
    for w, n_rows in ((big, 128), (small, 17)):
        p, (Q, K, V, O, rows) = _case(w, n_rows)
        n = rows.numel()
        ref = torch.full((p.B * p.H + 1,), -1.0, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(mcs.workspace_size(p, mcs.MCS_WS_DRIFT)[0], 1), dtype=torch.uint8, device="cuda")
        mcs.residual_drift(p, Q, K, V, O, rows, ref, ws)
        got = torch.full_like(ref, -2.0)
        mcs.residual_drift_noalloc(p, Q, K, V, O, rows, got)
        torch.cuda.synchronize()
        print(f"{w.name}: {n} rows, drift {got.cpu().numpy()}", flush=True)
        assert torch.equal(got, ref), (got, ref)
        assert np.all(np.isfinite(got.cpu().numpy())) and got[-1].item() == got[:-1].max().item()
    # a problem whose scratch exceeds the static array: refused before any launch
    p = mcs.problem(1, 40, 75600, 75600, 128, 128, 2268, dtype="bf16")
    out = torch.zeros(p.B * p.H + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(mcs.MCSError) as e:
        mcs.residual_drift_noalloc(p, Q, K, V, O, rows, out, n_rows=128)
    assert e.value.status == mcs.MCS_ERR_WORKSPACE
