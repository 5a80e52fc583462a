"""Device-resident synthetic inputs for a workload (plumbing, no attention math).

Heads are generated on host threads with ``synth.head_inputs`` (each head has
its own seeds) and copied into preallocated device tensors, so host memory
stays at a few heads regardless of the workload size.
"""
from __future__ import annotations

import concurrent.futures as cf
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

from . import synth


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _to_tensor(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def device_inputs(w: synth.Workload, step: int, device="cuda",
                  keep_heads: Iterable[Tuple[int, int]] = (), out=None):
    """Q, K, V of all heads at ``step`` on ``device`` ([B,H,N,d]); also returns
    the host float32 copies of the heads listed in ``keep_heads``.  ``out``
    may pass (Q, K, V) device tensors to fill in place."""
    import torch
    dt = torch_dtype(w)
    if out is None:
        Q = torch.empty((w.B, w.H, w.Nq, w.d), dtype=dt, device=device)
        K = torch.empty((w.B, w.H, w.Nkv, w.d), dtype=dt, device=device)
        V = torch.empty((w.B, w.H, w.Nkv, w.d), dtype=dt, device=device)
    else:
        Q, K, V = out
    keep = set(keep_heads)
    host: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def gen(bh):
        b, h = bh
        q, k, v = synth.head_inputs(w, b, h, step)
        if bh in keep:
            host[bh] = (q, k, v)
        return bh, (_to_tensor(q, w.dtype), _to_tensor(k, w.dtype), _to_tensor(v, w.dtype))

    with cf.ThreadPoolExecutor(synth._threads()) as ex:
        for (b, h), (q, k, v) in ex.map(gen, heads):
            Q[b, h].copy_(q)
            K[b, h].copy_(k)
            V[b, h].copy_(v)
    return (Q, K, V), host
