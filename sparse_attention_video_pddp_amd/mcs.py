"""ctypes binding of libmcs.so (the C ABI in include/mcs.h).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  PyTorch is used for device memory and the current stream; tensors
are passed as raw device pointers.  If the library has not been built the
import of this module still works, but every call raises (there is no CPU
fallback).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmcs.so")

MCS_OK, MCS_ERR_INVALID_ARG, MCS_ERR_UNSUPPORTED, MCS_ERR_WORKSPACE, MCS_ERR_HIP = range(5)
MCS_F32, MCS_BF16 = 0, 1
MCS_WS_GROUP, MCS_WS_ANCHOR, MCS_WS_BLOCK, MCS_WS_DRIFT = 0, 1, 2, 3
MCS_ANCHOR_AUTO, MCS_ANCHOR_TWO_PASS, MCS_ANCHOR_SINGLE_PASS = 0, 1, 2
_ANCHOR_MODES = {"auto": MCS_ANCHOR_AUTO, "two_pass": MCS_ANCHOR_TWO_PASS, "single_pass": MCS_ANCHOR_SINGLE_PASS}
MAX_DRIFT_ROWS = 128

EXPORTED = ("mcs_workspace_size", "mcs_group", "mcs_dense_attn", "mcs_anchor", "mcs_sparse_attn",
            "mcs_block_select", "mcs_residual_drift", "mcs_residual_drift_noalloc", "mcs_status_string",
            "mcs_last_error", "mcs_version")


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nkv", ctypes.c_int32), ("d", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("k", ctypes.c_int32), ("scale", ctypes.c_float), ("causal_block", ctypes.c_int32),
                ("q_offset", ctypes.c_int32), ("pddp_iters", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("r_dtype", ctypes.c_int32), ("anchor_mode", ctypes.c_int32)]

    def __repr__(self) -> str:
        return "Problem(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"

    @property
    def n_groups(self) -> int:
        return -(-self.Nq // self.group_size)


class MCSError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def _status_name(s: int) -> str:
    names = {0: "MCS_OK", 1: "MCS_ERR_INVALID_ARG", 2: "MCS_ERR_UNSUPPORTED", 3: "MCS_ERR_WORKSPACE",
             4: "MCS_ERR_HIP"}
    return names.get(s, f"status {s}")


def lib() -> ctypes.CDLL:
    """Load libmcs.so (in-tree build).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_video_pddp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.mcs_workspace_size.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.mcs_group.argtypes = [P, vp, vp, vp, sz, vp]
        L.mcs_dense_attn.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.mcs_anchor.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mcs_sparse_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.mcs_block_select.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.mcs_residual_drift.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, sz, vp]
        L.mcs_residual_drift_noalloc.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp]
        for f in ("mcs_workspace_size", "mcs_group", "mcs_dense_attn", "mcs_anchor", "mcs_sparse_attn",
                  "mcs_block_select", "mcs_residual_drift", "mcs_residual_drift_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.mcs_status_string.argtypes = [ctypes.c_int]
        L.mcs_status_string.restype = ctypes.c_char_p
        L.mcs_last_error.argtypes = []
        L.mcs_last_error.restype = ctypes.c_char_p
        L.mcs_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MCS_OK:
        raise MCSError(status, lib().mcs_last_error().decode())


_DTYPES = {"f32": MCS_F32, "bf16": MCS_BF16}


def problem(B: int, H: int, Nq: int, Nkv: int, d: int, group_size: int, k: int, scale: Optional[float] = None,
            causal_block: int = 0, q_offset: int = 0, pddp_iters: int = 32, dtype: str = "bf16",
            r_dtype: str = "f32", anchor_mode: str = "auto") -> Problem:
    """Problem description; the residual R is float32 unless r_dtype="bf16"
    (bf16 problems only); anchor_mode "auto", "two_pass" or "single_pass"."""
    return Problem(B, H, Nq, Nkv, d, group_size, k, 1.0 / math.sqrt(d) if scale is None else scale,
                   causal_block, q_offset, pddp_iters, _DTYPES[dtype], _DTYPES[r_dtype], _ANCHOR_MODES[anchor_mode])


def problem_for(w, r_dtype: str = "f32", anchor_mode: str = "auto") -> Problem:
    """Problem of a synthetic workload (``synth.Workload``)."""
    return problem(w.B, w.H, w.Nq, w.Nkv, w.d, w.group_size, w.k, w.scale, w.causal_block, w.q_offset,
                   w.pddp_iters, w.dtype, r_dtype, anchor_mode)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _torch_stream(stream):
    """The torch stream object for a ``stream`` argument (None: the current
    stream; an int: a raw hipStream_t handle)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def workspace_size(p: Problem, kind: int) -> Tuple[int, int]:
    b, m = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mcs_workspace_size(ctypes.byref(p), kind, ctypes.byref(b), ctypes.byref(m)))
    return b.value, m.value


def group(p: Problem, Q, perm, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().mcs_group(ctypes.byref(p), _ptr(Q), _ptr(perm), _ptr(ws), nbytes, _stream(stream)))


def dense_attn(p: Problem, Q, K, V, O, lse=None, stream=None) -> None:
    _check(lib().mcs_dense_attn(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                                _stream(stream)))


def anchor(p: Problem, Q, K, V, perm, O, idx, R, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().mcs_anchor(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(perm), _ptr(O), _ptr(idx),
                            _ptr(R), _ptr(ws), nbytes, _stream(stream)))


def sparse_attn(p: Problem, Q, K, V, perm, idx, R, O, stream=None) -> None:
    _check(lib().mcs_sparse_attn(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(perm), _ptr(idx), _ptr(R),
                                 _ptr(O), _stream(stream)))


def block_select(p: Problem, Q, K, perm, idx, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().mcs_block_select(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(perm), _ptr(idx), _ptr(ws), nbytes,
                                  _stream(stream)))


def residual_drift(p: Problem, Q, K, V, O, rows, drift, ws, n_rows: Optional[int] = None,
                   ws_bytes: Optional[int] = None, stream=None) -> None:
    """drift: B*H + 1 float32 values, the per-head drifts then their maximum."""
    if hasattr(drift, "numel") and drift.numel() < p.B * p.H + 1:
        raise ValueError(f"drift holds {drift.numel()} values; B*H + 1 = {p.B * p.H + 1} are written")
    n = rows.numel() if n_rows is None else n_rows
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().mcs_residual_drift(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(rows), n,
                                    _ptr(drift), _ptr(ws), nbytes, _stream(stream)))


def residual_drift_noalloc(p: Problem, Q, K, V, O, rows, drift, n_rows: Optional[int] = None, stream=None) -> None:
    """mcs_residual_drift without a workspace: the library's static scratch
    (for callers that cannot allocate; calls overlapping on one GPU race)."""
    if hasattr(drift, "numel") and drift.numel() < p.B * p.H + 1:
        raise ValueError(f"drift holds {drift.numel()} values; B*H + 1 = {p.B * p.H + 1} are written")
    n = rows.numel() if n_rows is None else n_rows
    _check(lib().mcs_residual_drift_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(rows), n,
                                            _ptr(drift), _stream(stream)))


class MCSparseAttention:
    """Per-layer state of the method across denoising steps: the groups
    (perm), selections (idx) and residual (R) of the last anchor, held in
    device tensors, plus the two workspaces.  ``step(Q, K, V, is_anchor)``
    runs grouping + anchor or the reuse step and returns O."""

    def __init__(self, p: Problem, device="cuda"):
        import torch
        self.p = p
        dt = torch.bfloat16 if p.dtype == MCS_BF16 else torch.float32
        BH = p.B * p.H
        self.perm = torch.empty((p.B, p.H, p.Nq), dtype=torch.int32, device=device)
        self.idx = torch.empty((p.B, p.H, p.n_groups, p.k), dtype=torch.int32, device=device)
        rdt = torch.bfloat16 if p.r_dtype == MCS_BF16 else torch.float32
        self.R = torch.empty((p.B, p.H, p.Nq, p.d), dtype=rdt, device=device)  # float32 unless asked for bf16
        self.O = torch.empty((p.B, p.H, p.Nq, p.d), dtype=dt, device=device)
        g, _ = workspace_size(p, MCS_WS_GROUP)
        a, _ = workspace_size(p, MCS_WS_ANCHOR)
        self.ws_group = torch.empty(max(g, 1), dtype=torch.uint8, device=device)
        self.ws_anchor = torch.empty(max(a, 1), dtype=torch.uint8, device=device)
        self.has_anchor = BH == 0

    def step(self, Q, K, V, is_anchor: bool, stream=None):
        if is_anchor:
            group(self.p, Q, self.perm, self.ws_group, stream=stream)
            anchor(self.p, Q, K, V, self.perm, self.O, self.idx, self.R, self.ws_anchor, stream=stream)
            self.has_anchor = True
        else:
            if not self.has_anchor:
                raise RuntimeError("a reuse step needs a previous anchor step")
            sparse_attn(self.p, Q, K, V, self.perm, self.idx, self.R, self.O, stream=stream)
        return self.O


class BlockSparseComparator:
    """The block-sparse comparator at the same token budget k: the mean-pooled
    block selection recomputed from every step's Q/K, then attention over the
    selected tokens with no residual.  ``step(Q, K, V)`` returns O."""

    def __init__(self, p: Problem, device="cuda"):
        import torch
        self.p = p
        dt = torch.bfloat16 if p.dtype == MCS_BF16 else torch.float32
        self.perm = torch.empty((p.B, p.H, p.Nq), dtype=torch.int32, device=device)
        self.idx = torch.empty((p.B, p.H, p.n_groups, p.k), dtype=torch.int32, device=device)
        self.O = torch.empty((p.B, p.H, p.Nq, p.d), dtype=dt, device=device)
        b, _ = workspace_size(p, MCS_WS_BLOCK)
        self.ws = torch.empty(max(b, 1), dtype=torch.uint8, device=device)

    def step(self, Q, K, V, stream=None):
        block_select(self.p, Q, K, self.perm, self.idx, self.ws, stream=stream)
        sparse_attn(self.p, Q, K, V, self.perm, self.idx, None, self.O, stream=stream)
        return self.O


def drift_rows(Nq: int, n: int = MAX_DRIFT_ROWS):
    """n query rows spread evenly over [0, Nq) (fewer if Nq < n), as a host list."""
    n = max(1, min(n, Nq, MAX_DRIFT_ROWS))
    return sorted({(2 * i + 1) * Nq // (2 * n) for i in range(n)})


class AdaptiveAnchoring:
    """Anchor schedule driven by the residual-drift check instead of a fixed
    period: after every reuse step the drift of the sampled rows is measured
    (mcs_residual_drift on the step's output), and the next step is an anchor
    when the largest drift over the heads exceeds ``threshold`` or when
    ``max_period`` steps have passed since the last anchor (0: no limit).
    ``step(Q, K, V)`` returns O; ``history`` records (is_anchor, drift) per
    step.  Reading the drift back costs one host synchronisation per reuse
    step; the read is ordered after the check on the stream it ran on."""

    def __init__(self, layer: MCSparseAttention, threshold: float, max_period: int = 0, n_rows: int = 64,
                 device="cuda"):
        import torch
        self.layer, self.threshold, self.max_period = layer, threshold, max_period
        p = layer.p
        self.rows = torch.tensor(drift_rows(p.Nq, n_rows), dtype=torch.int32, device=device)
        self.drift = torch.zeros(p.B * p.H + 1, dtype=torch.float32, device=device)  # per head, then the max
        b, _ = workspace_size(p, MCS_WS_DRIFT)
        self.ws = torch.empty(max(b, 1), dtype=torch.uint8, device=device)
        self.anchor_next = True
        self.since = 0
        self.history = []

    @staticmethod
    def decide(drift_max: float, threshold: float, since: int, max_period: int) -> bool:
        """Whether the step after a reuse step with this drift is an anchor
        (a NaN drift anchors too)."""
        return not (drift_max <= threshold) or (max_period > 0 and since + 1 >= max_period)

    def step(self, Q, K, V, stream=None):
        if self.anchor_next or not self.layer.has_anchor:
            O = self.layer.step(Q, K, V, True, stream=stream)
            self.anchor_next, self.since = False, 0
            self.history.append((True, None))
            return O
        O = self.layer.step(Q, K, V, False, stream=stream)
        residual_drift(self.layer.p, Q, K, V, O, self.rows, self.drift, self.ws, stream=stream)
        import torch
        with torch.cuda.stream(_torch_stream(stream)):
            d = self.drift[-1].item()  # the largest drift over the heads, computed by the library
        self.since += 1
        self.anchor_next = self.decide(d, self.threshold, self.since, self.max_period)
        self.history.append((False, d))
        return O


class ChunkedCausalStream:
    """Chunked autoregressive generation over a K/V cache: the video is made
    chunk by chunk (``frames_per_chunk`` frames of ``frame_tokens`` tokens),
    each chunk denoised over several steps while it attends, frame-block
    causally, to the finished chunks and to itself.

    The cache holds the K and V rows of the whole video, [B,H,capacity,d],
    zero where nothing has been generated yet; chunk c's queries sit at
    positions c*chunk_tokens.. of it.  Every chunk is an ordinary problem with
    Nkv = capacity, q_offset = c*chunk_tokens and causal_block = frame_tokens:
    keys past the chunk's last frame are invisible, so neither the cache's
    unwritten rows nor its size change any result (they must only be finite,
    hence the zeros).  Grouping, selections and residual are per chunk (a
    fresh ``MCSparseAttention`` in ``begin_chunk``); the anchor schedule inside
    a chunk is the caller's.  ``step`` writes the chunk's current K/V rows
    into the cache (or the caller fills ``kv_rows()`` in place) and runs the
    step, all on ``stream``, which first waits for the current stream (where
    the caller made the chunk's rows)."""

    def __init__(self, B: int, H: int, d: int, frame_tokens: int, frames_per_chunk: int, n_chunks: int,
                 group_size: int, k: int, scale: Optional[float] = None, dtype: str = "bf16",
                 pddp_iters: int = 32, device="cuda", r_dtype: str = "f32", anchor_mode: str = "auto"):
        import torch
        self.B, self.H, self.d = B, H, d
        self.frame_tokens = frame_tokens
        self.chunk_tokens = frame_tokens * frames_per_chunk
        self.n_chunks = n_chunks
        self.capacity = self.chunk_tokens * n_chunks
        self.G, self.k, self.scale, self.dtype, self.iters = group_size, k, scale, dtype, pddp_iters
        self.r_dtype, self.anchor_mode = r_dtype, anchor_mode
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.K = torch.zeros((B, H, self.capacity, d), dtype=dt, device=device)
        self.V = torch.zeros_like(self.K)
        self.device = device
        self.chunk = -1
        self.layer: Optional[MCSparseAttention] = None

    def problem(self, c: int) -> Problem:
        return problem(self.B, self.H, self.chunk_tokens, self.capacity, self.d, self.G, self.k, self.scale,
                       causal_block=self.frame_tokens, q_offset=c * self.chunk_tokens, pddp_iters=self.iters,
                       dtype=self.dtype, r_dtype=self.r_dtype, anchor_mode=self.anchor_mode)

    def rows(self, c: Optional[int] = None) -> slice:
        c = self.chunk if c is None else c
        return slice(c * self.chunk_tokens, (c + 1) * self.chunk_tokens)

    def begin_chunk(self) -> Problem:
        if self.chunk + 1 >= self.n_chunks:
            raise RuntimeError("the stream's capacity is used up")
        self.chunk += 1
        self.layer = MCSparseAttention(self.problem(self.chunk), device=self.device)
        return self.layer.p

    def kv_rows(self):
        """Views of the current chunk's K and V rows in the cache."""
        r = self.rows()
        return self.K[:, :, r], self.V[:, :, r]

    def step(self, Q, K_chunk=None, V_chunk=None, is_anchor: bool = False, stream=None):
        if self.layer is None:
            raise RuntimeError("begin_chunk() first")
        import torch
        ts = _torch_stream(stream)
        cur = torch.cuda.current_stream()
        if ts != cur:
            ts.wait_stream(cur)
        if K_chunk is not None:
            k, v = self.kv_rows()
            with torch.cuda.stream(ts):
                k.copy_(K_chunk)
                v.copy_(V_chunk)
            if ts != cur:
                # the caller may free the chunk's rows once this returns: keep the
                # allocator from handing their memory out before ts has read them
                K_chunk.record_stream(ts)
                V_chunk.record_stream(ts)
        return self.layer.step(Q, self.K, self.V, is_anchor, stream=ts)
