"""Run a synthetic workload through the C ABI on the GPU and collect the
sampled heads' inputs and outputs for the staged parity checks."""
from __future__ import annotations

import sys
from typing import Dict, Iterable, Sequence, Tuple

import numpy as np

from sparse_attention_video_pddp_amd import mcs, synth
from sparse_attention_video_pddp_amd.workload import device_inputs
from tests.parity import HeadCase


def _np(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_anchor_reuse(w: synth.Workload, heads: Sequence[Tuple[int, int]], anchor_step: int = 0,
                     reuse_step: int = 1, r_dtype: str = "f32", anchor_mode: str = "auto"
                     ) -> Dict[Tuple[int, int], HeadCase]:
    """mcs_group + mcs_anchor on the anchor step's inputs, then mcs_sparse_attn
    on the reuse step's inputs (residual stored in r_dtype, selections made
    in anchor_mode); returns HeadCase per sampled (b, h)."""
    import torch
    p = mcs.problem_for(w, r_dtype, anchor_mode)
    log(f"[gpu] {w.name}: {p}")
    (Q0, K0, V0), h0 = device_inputs(w, anchor_step, keep_heads=heads)
    state = mcs.MCSparseAttention(p)
    O_full = state.step(Q0, K0, V0, True).clone()
    torch.cuda.synchronize()
    del Q0, K0, V0
    (Q1, K1, V1), h1 = device_inputs(w, reuse_step, keep_heads=heads)
    O_re = state.step(Q1, K1, V1, False)
    torch.cuda.synchronize()
    out = {}
    for (b, h) in heads:
        q0, k0, v0 = (x.astype(np.float64) for x in h0[(b, h)])
        q1, k1, v1 = (x.astype(np.float64) for x in h1[(b, h)])
        out[(b, h)] = HeadCase(q0, k0, v0, q1, k1, v1,
                               perm=_np(state.perm[b, h]), idx=_np(state.idx[b, h]),
                               O_full=_np(O_full[b, h]).astype(np.float64),
                               R=_np(state.R[b, h]).astype(np.float64),
                               O_reuse=_np(O_re[b, h]).astype(np.float64))
    return out
