"""Seeded synthetic video-token workloads (inputs only; no attention arithmetic).

The pages evaluate MC-Sparse on video and 3D-asset diffusion transformers whose
weights are not available here, so every workload is synthetic: Q/K/V shaped
like a 3D (frame x height x width) latent, with the spatial structure that
makes token-level selection meaningful.

* Fourier-structured generator: a random Fourier feature F(t, y, x) of the
  integer grid coordinates (Rahimi-Recht features: Gaussian frequencies,
  uniform phases, amplitude sqrt(2) so each component has unit variance),
  Q = 0.7 F + 0.3 eps', K = 0.7 F + 0.3 eps, V ~ N(0, 1).  Neighbouring tokens
  have correlated features, which is the locality the MonarchRT summary
  describes for 3D attention maps (MonarchRT page, section 2: periodic
  positional structure plus sparse semantic links).
* 3D-local generator: per head and channel, white noise on the grid smoothed
  by a periodic Gaussian (sigma in cells) and rescaled to unit variance;
  Q and K add independent 0.2 N(0, 1) noise.
* Drift between denoising steps: a cumulative random walk
  X_{t+1} = X_t + sigma N(0, 1) for each of Q, K, V.
* Optional query offset (test workloads only): Q += q_mean * m with
  m_c = 1 + 0.5 z_c, z ~ N(0, 1) per head and channel, i.e. a mean shared by
  every query along the all-ones direction plus a per-channel spread, tens of
  times the queries' own spread.  Grouping must centre each node on its mean;
  this makes any loss of precision in that step visible.

Tokens are flattened frame-major, n = (t * height + y) * width + x, following
the per-axis (f, h, w) block alignment in the MonarchRT summary (section 2).

Every random draw comes from ``numpy.random.SeedSequence([cfg_id, role,
b*H + h, step])`` so that any single head at any step can be regenerated on its
own (the parity tests regenerate sampled heads).  bf16 inputs are produced by
rounding the fp32 values once, round-to-nearest-even; the HIP path and the
oracle both consume exactly those values.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

# Roles in the seed tuple.  Fixed numbering: changing it changes every input.
ROLE_W, ROLE_PHASE, ROLE_EPS_Q, ROLE_EPS_K, ROLE_V = 0, 1, 2, 3, 4
ROLE_DRIFT_Q, ROLE_DRIFT_K, ROLE_DRIFT_V = 5, 6, 7
ROLE_FIELD, ROLE_NOISE_Q, ROLE_NOISE_K = 8, 9, 10
ROLE_Q_MEAN = 11


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload (shapes, method parameters, inputs recipe)."""

    name: str
    cfg_id: int                 # seed namespace
    B: int
    H: int
    grid: Tuple[int, int, int]  # (frames, height, width) of the KV sequence
    d: int
    dtype: str                  # "bf16" or "f32"
    group_size: int             # G
    keep_permille: int          # keep fraction in per-mille
    scale: float                # logit multiplier
    causal_block: int = 0       # 0: bidirectional; else tokens per causal block
    q_frames: Optional[Tuple[int, int]] = None  # query chunk [t0, t1) of the grid
    generator: str = "fourier"  # "fourier" or "field"
    fourier_mix: Tuple[float, float] = (0.7, 0.3)
    field_sigma: float = 2.0
    field_noise: float = 0.2
    drift: float = 0.03
    q_mean: float = 0.0         # common query offset (see head_base); 0 for the benchmark workloads
    steps: int = 2
    anchor_every: int = 1 << 30
    pddp_iters: int = 32

    # ---- derived sizes ------------------------------------------------------
    @property
    def Nkv(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def Nq(self) -> int:
        if self.q_frames is None:
            return self.Nkv
        t0, t1 = self.q_frames
        return (t1 - t0) * self.grid[1] * self.grid[2]

    @property
    def q_offset(self) -> int:
        """Position of query 0 inside the KV sequence."""
        if self.q_frames is None:
            return 0
        return self.q_frames[0] * self.grid[1] * self.grid[2]

    @property
    def k(self) -> int:
        """KV tokens kept per group: ceil(Nkv * keep) in integer arithmetic."""
        return (self.Nkv * self.keep_permille + 999) // 1000

    @property
    def n_groups(self) -> int:
        return -(-self.Nq // self.group_size)

    def is_anchor(self, step: int) -> bool:
        return step % self.anchor_every == 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(**kw) -> Workload:
    return Workload(**kw)


# The five workloads, in the order they are listed for this method's
# benchmark (tiny smoke test; chunked causal; full bidirectional at 5% and
# 10%; large latent; long-sequence stress).
CONFIGS: Dict[str, Workload] = {
    "tiny": _wl(name="tiny", cfg_id=1, B=1, H=2, grid=(4, 16, 16), d=64, dtype="f32",
                group_size=64, keep_permille=100, scale=2.0 / math.sqrt(64),
                drift=0.05, steps=2, anchor_every=2),
    "causal": _wl(name="causal", cfg_id=2, B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
                  group_size=64, keep_permille=50, scale=1.0 / math.sqrt(128),
                  causal_block=30 * 52, q_frames=(18, 21), drift=0.03, steps=8,
                  anchor_every=4),
    "bidir5": _wl(name="bidir5", cfg_id=3, B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
                  group_size=64, keep_permille=50, scale=1.0 / math.sqrt(128),
                  drift=0.03, steps=10, anchor_every=5),
    "bidir10": _wl(name="bidir10", cfg_id=3, B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
                   group_size=64, keep_permille=100, scale=1.0 / math.sqrt(128),
                   drift=0.03, steps=10, anchor_every=5),
    "large": _wl(name="large", cfg_id=4, B=1, H=40, grid=(21, 45, 80), d=128, dtype="bf16",
                 group_size=128, keep_permille=30, scale=3.0 / math.sqrt(128),
                 drift=0.03, steps=10, anchor_every=5),
    "stress": _wl(name="stress", cfg_id=5, B=1, H=16, grid=(32, 64, 64), d=64, dtype="bf16",
                  group_size=128, keep_permille=20, scale=1.0 / math.sqrt(64),
                  generator="field", drift=0.03, steps=6, anchor_every=3),
}


def get(name: str, **overrides) -> Workload:
    w = CONFIGS[name]
    return w.with_(**overrides) if overrides else w


# ---------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ---------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value (returned as fp32)."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------------------
# Per-head generation
# ---------------------------------------------------------------------------
def _rng(w: Workload, role: int, bh: int, step: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cfg_id, role, bh, step])))


def grid_coords(grid: Tuple[int, int, int], frames: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Integer (t, y, x) coordinates in frame-major token order, shape [N, 3]."""
    T, Hg, Wg = grid
    t0, t1 = frames if frames is not None else (0, T)
    t, y, x = np.meshgrid(np.arange(t0, t1), np.arange(Hg), np.arange(Wg), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)


def _fourier_features(w: Workload, bh: int, coords: np.ndarray) -> np.ndarray:
    W = _rng(w, ROLE_W, bh, 0).standard_normal((w.d, 3))
    phase = _rng(w, ROLE_PHASE, bh, 0).uniform(0.0, 2.0 * math.pi, size=w.d)
    return math.sqrt(2.0) * np.cos(coords @ W.T + phase[None, :])


def _smoothed_field(w: Workload, bh: int) -> np.ndarray:
    T, Hg, Wg = w.grid
    noise = _rng(w, ROLE_FIELD, bh, 0).standard_normal((w.d, T, Hg, Wg))
    ft = np.fft.fftfreq(T)[:, None, None]
    fy = np.fft.fftfreq(Hg)[None, :, None]
    fx = np.fft.rfftfreq(Wg)[None, None, :]
    s = w.field_sigma
    transfer = np.exp(-2.0 * math.pi ** 2 * s * s * (ft * ft + fy * fy + fx * fx))
    field = np.fft.irfftn(np.fft.rfftn(noise, axes=(1, 2, 3)) * transfer[None], s=(T, Hg, Wg),
                          axes=(1, 2, 3))
    field = field.reshape(w.d, -1)
    field -= field.mean(axis=1, keepdims=True)
    field /= field.std(axis=1, keepdims=True)
    return field.T  # [N, d]


def head_base(w: Workload, b: int, h: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Step-0 Q [Nq,d], K [Nkv,d], V [Nkv,d] for one (b, h), float64."""
    bh = b * w.H + h
    if w.generator == "fourier":
        a, e = w.fourier_mix
        Fk = _fourier_features(w, bh, grid_coords(w.grid))
        if w.q_frames is None:
            Fq = Fk
        else:
            Fq = _fourier_features(w, bh, grid_coords(w.grid, w.q_frames))
        Q = a * Fq + e * _rng(w, ROLE_EPS_Q, bh, 0).standard_normal(Fq.shape)
        K = a * Fk + e * _rng(w, ROLE_EPS_K, bh, 0).standard_normal(Fk.shape)
    elif w.generator == "field":
        if w.q_frames is not None:
            raise ValueError("the 3D-local generator has no query chunk form")
        field = _smoothed_field(w, bh)
        Q = field + w.field_noise * _rng(w, ROLE_NOISE_Q, bh, 0).standard_normal(field.shape)
        K = field + w.field_noise * _rng(w, ROLE_NOISE_K, bh, 0).standard_normal(field.shape)
    else:
        raise ValueError(f"unknown generator {w.generator!r}")
    if w.q_mean:
        m = 1.0 + 0.5 * _rng(w, ROLE_Q_MEAN, bh, 0).standard_normal(w.d)
        Q = Q + w.q_mean * m[None, :]
    V = _rng(w, ROLE_V, bh, 0).standard_normal((w.Nkv, w.d))
    return Q, K, V


def head_inputs(w: Workload, b: int, h: int, step: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of one (b, h) at a denoising step, as float32 in the compute dtype's values.

    For bf16 workloads the values are already rounded to bf16 (exactly
    representable), so ``bf16_bits`` of them is lossless.
    """
    Q, K, V = head_base(w, b, h)
    bh = b * w.H + h
    for t in range(1, step + 1):
        Q = Q + w.drift * _rng(w, ROLE_DRIFT_Q, bh, t).standard_normal(Q.shape)
        K = K + w.drift * _rng(w, ROLE_DRIFT_K, bh, t).standard_normal(K.shape)
        V = V + w.drift * _rng(w, ROLE_DRIFT_V, bh, t).standard_normal(V.shape)
    out = []
    for X in (Q, K, V):
        X = X.astype(np.float32)
        if w.dtype == "bf16":
            X = round_bf16(X)
        out.append(X)
    return out[0], out[1], out[2]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def step_inputs(w: Workload, step: int, heads: Optional[Iterable[Tuple[int, int]]] = None
                ) -> Dict[str, np.ndarray]:
    """All heads' Q/K/V at one step as float32 arrays [B,H,N,d].

    ``heads`` restricts generation to the listed (b, h) pairs (others stay 0).
    Heads are generated in a thread pool; every head uses its own seeds, so
    the result does not depend on the thread count.
    """
    Q = np.zeros((w.B, w.H, w.Nq, w.d), np.float32)
    K = np.zeros((w.B, w.H, w.Nkv, w.d), np.float32)
    V = np.zeros((w.B, w.H, w.Nkv, w.d), np.float32)
    todo = list(heads) if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        q, k, v = head_inputs(w, b, h, step)
        Q[b, h], K[b, h], V[b, h] = q, k, v

    if len(todo) == 1:
        one(todo[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, todo))
    return {"Q": Q, "K": K, "V": V}


def to_device_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Host array in the wire format the library consumes (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)
