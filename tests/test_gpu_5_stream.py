"""GPU parity of chunked-causal streaming (ChunkedCausalStream) against the
fp64 oracle.

A small video is generated chunk by chunk over a zero-initialised K/V cache
of the whole video: each chunk of two frames runs an anchor step and two
reuse steps with drifting inputs, its K/V rows written into the cache, the
finished chunks' rows staying as their last step left them.  Every chunk is
checked like a single workload (grouping, dense rows, top-k, residual and
reuse output of every head, tests/parity.py), with the oracle given the same
cache (its unwritten rows are invisible to the chunk's queries), plus the
second reuse step.  Inputs: the frame-causal workload's Fourier generator on
an 8 x 10 x 15 grid, the chunk's queries and K/V rows from the generator of
that chunk.
"""
import numpy as np
import pytest

from oracle import mcs_oracle as orc
from sparse_attention_video_pddp_amd import synth
from tests.parity import HeadCase, assert_reports, check_head, compare

pytestmark = pytest.mark.gpu

FPC, T, HGT, WID = 2, 8, 10, 15          # frames per chunk, frames, height, width
BASE = synth.get("causal").with_(name="stream_small", H=2, grid=(T, HGT, WID), causal_block=HGT * WID,
                                 keep_permille=80)


@pytest.fixture(scope="module")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def test_chunked_causal_stream_parity(cuda):
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import _to_tensor
    from tests.gpu_runner import log
    ft = HGT * WID
    n_chunks = T // FPC
    w0 = BASE.with_(q_frames=(0, FPC))
    st = mcs.ChunkedCausalStream(w0.B, w0.H, w0.d, ft, FPC, n_chunks, w0.group_size, w0.k, w0.scale, w0.dtype,
                                 w0.pddp_iters)
    cache_k = np.zeros((w0.H, st.capacity, w0.d), np.float32)   # host mirror (B = 1)
    cache_v = np.zeros_like(cache_k)
    for c in range(n_chunks):
        wc = BASE.with_(q_frames=(c * FPC, (c + 1) * FPC))
        p = st.begin_chunk()
        assert (p.Nq, p.Nkv, p.q_offset, p.causal_block) == (wc.Nq, st.capacity, wc.q_offset, ft)
        r = st.rows()
        steps = []
        for s in range(3):
            qs, ks, vs = [], [], []
            for h in range(wc.H):
                q, k, v = synth.head_inputs(wc, 0, h, s)
                qs.append(q)
                ks.append(k[r])
                vs.append(v[r])
                cache_k[h, r], cache_v[h, r] = k[r], v[r]
            dev = [torch.stack([_to_tensor(x, wc.dtype) for x in xs])[None].to("cuda") for xs in (qs, ks, vs)]
            O = st.step(dev[0], dev[1], dev[2], is_anchor=(s == 0)).clone()
            torch.cuda.synchronize()
            steps.append((qs, cache_k.copy(), cache_v.copy(), O,
                          st.layer.perm.clone(), st.layer.idx.clone(), st.layer.R.clone()))
        (q0, k0, v0, O0, perm, idx, R), (q1, k1, v1, O1, *_), (q2, k2, v2, O2, *_) = steps
        for h in range(wc.H):
            f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
            case = HeadCase(f64(q0[h]), f64(k0[h]), f64(v0[h]), f64(q1[h]), f64(k1[h]), f64(v1[h]),
                            perm=perm[0, h].cpu().numpy(), idx=idx[0, h].cpu().numpy(),
                            O_full=O0[0, h].float().cpu().numpy().astype(np.float64),
                            R=R[0, h].float().cpu().numpy().astype(np.float64),
                            O_reuse=O1[0, h].float().cpu().numpy().astype(np.float64))
            reps = check_head(case, wc.group_size, wc.k, wc.scale, ft, wc.q_offset, wc.pddp_iters)
            # second reuse step on the same groups, selections and residual
            ref2 = orc.reuse_step(f64(q2[h]), f64(k2[h]), f64(v2[h]), case.perm, case.idx, case.R,
                                  wc.group_size, wc.scale, ft, wc.q_offset)
            reps.append(compare("O (second reuse step)", O2[0, h].float().cpu().numpy(), ref2,
                                float(np.abs(v2[h]).max())))
            for rep in reps:
                log(f"  chunk {c} head {h}: {rep}")
            assert_reports(reps, f"chunk {c} head {h}")
    # every row of the cache was written once, and nothing past it
    assert np.array_equal(st.K[0].float().cpu().numpy(), cache_k)
    with pytest.raises(RuntimeError):
        st.begin_chunk()


def test_chunked_stream_on_a_side_stream(cuda):
    """ChunkedCausalStream handed a side stream without a stream context: the
    chunk's K/V rows are copied into the cache on that stream after it waits
    for the current one (where they were made), so every output and the cache
    equal those of the current stream bit for bit."""
    import torch
    from sparse_attention_video_pddp_amd import mcs
    from sparse_attention_video_pddp_amd.workload import _to_tensor
    ft = HGT * WID
    n_chunks = T // FPC

    def run(stream):
        w0 = BASE.with_(q_frames=(0, FPC))
        st = mcs.ChunkedCausalStream(w0.B, w0.H, w0.d, ft, FPC, n_chunks, w0.group_size, w0.k, w0.scale,
                                     w0.dtype, w0.pddp_iters)
        outs = []
        for c in range(2):
            wc = BASE.with_(q_frames=(c * FPC, (c + 1) * FPC))
            st.begin_chunk()
            r = st.rows()
            for s in range(2):
                hs = [synth.head_inputs(wc, 0, h, s) for h in range(wc.H)]
                dev = [torch.stack([_to_tensor(x[i] if i == 0 else x[i][r], wc.dtype) for x in hs])[None]
                       .to("cuda") for i in range(3)]
                O = st.step(dev[0], dev[1], dev[2], is_anchor=(s == 0), stream=stream)
                (stream or torch.cuda.current_stream()).synchronize()
                outs.append(O.clone())
        return outs, st.K.clone(), st.V.clone()

    ref = run(None)
    side = run(torch.cuda.Stream())
    for a, b in zip(ref[0], side[0]):
        assert torch.equal(a, b)
    assert torch.equal(ref[1], side[1]) and torch.equal(ref[2], side[2])
