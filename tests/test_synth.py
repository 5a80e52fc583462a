"""Generator determinism, sizes and statistics (not gpu)."""
import numpy as np
import pytest
import torch

from sparse_attention_video_pddp_amd import synth


def test_config_sizes_and_integer_keep():
    c = synth.CONFIGS
    assert (c["tiny"].Nq, c["tiny"].Nkv, c["tiny"].k, c["tiny"].n_groups) == (1024, 1024, 103, 16)
    assert (c["causal"].Nq, c["causal"].Nkv, c["causal"].k, c["causal"].q_offset) == (4680, 32760, 1638, 28080)
    assert c["causal"].n_groups == 74 and c["causal"].causal_block == 1560
    assert (c["bidir5"].Nq, c["bidir5"].k, c["bidir5"].n_groups) == (32760, 1638, 512)
    assert c["bidir10"].k == 3276
    assert (c["large"].Nq, c["large"].k, c["large"].n_groups) == (75600, 2268, 591)
    assert (c["stress"].Nq, c["stress"].k, c["stress"].n_groups) == (131072, 2622, 1024)
    assert [s for s in range(10) if c["bidir5"].is_anchor(s)] == [0, 5]
    assert [s for s in range(8) if c["causal"].is_anchor(s)] == [0, 4]
    assert [s for s in range(6) if c["stress"].is_anchor(s)] == [0, 3]


def test_bf16_rounding_is_nearest_even_and_matches_torch():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9, -2.5e-3, 3.3e4,
                  1e-30, -0.0], np.float32)
    r = synth.round_bf16(x)
    assert r[1] == 1.0                      # tie -> even (down)
    assert r[2] == 1.0 + 2 ** -6            # tie -> even (up)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, ref)
    rng = np.random.default_rng(0)
    y = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits(y), ref)
    np.testing.assert_array_equal(synth.round_bf16(synth.round_bf16(y)), synth.round_bf16(y))


def test_heads_regenerate_identically_and_independently():
    w = synth.get("tiny")
    full = synth.step_inputs(w, 1)
    one = synth.step_inputs(w, 1, heads=[(0, 1)])
    for n in "QKV":
        np.testing.assert_array_equal(full[n][0, 1], one[n][0, 1])
        assert not np.array_equal(full[n][0, 0], full[n][0, 1])
    q, k, v = synth.head_inputs(w, 0, 1, 1)
    np.testing.assert_array_equal(q, full["Q"][0, 1])


def test_fourier_statistics_and_drift():
    w = synth.get("bidir5").with_(H=1, grid=(6, 10, 12))
    q0, k0, v0 = synth.head_inputs(w, 0, 0, 0)
    q1, k1, v1 = synth.head_inputs(w, 0, 0, 1)
    assert q0.shape == (720, 128) and v0.shape == (720, 128)
    # Q = 0.7 F + 0.3 eps: per-component variance 0.49 + 0.09
    assert abs(q0.var() - 0.58) < 0.05 and abs(v0.var() - 1.0) < 0.05
    # bf16 values
    np.testing.assert_array_equal(q0, synth.round_bf16(q0))
    # drift 0.03 N(0,1), up to bf16 rounding
    assert abs((v1 - v0).std() - 0.03) < 0.005
    # locality: neighbouring tokens have more similar keys than distant ones
    near = np.mean(np.sum(k0[:-1] * k0[1:], axis=1))
    far = np.mean(np.sum(k0[:360] * k0[360:], axis=1))
    assert near > 3 * abs(far)


def test_causal_queries_use_the_last_frames():
    w = synth.get("causal").with_(H=1, grid=(5, 6, 8), q_frames=(3, 5))
    assert w.Nq == 96 and w.q_offset == 144
    q, k, _ = synth.head_inputs(w, 0, 0, 0)
    # same features: query n and key q_offset + n share F, so they correlate strongly
    assert np.mean(np.sum(q * k[144:], axis=1)) > 0.3 * 128


def test_field_generator_statistics():
    w = synth.get("stress").with_(H=1, grid=(8, 16, 16))
    q, k, v = synth.head_inputs(w, 0, 0, 0)
    assert q.shape == (2048, 64)
    assert abs(q.var() - 1.04) < 0.08
    # smooth field: adjacent x tokens correlate ~exp(-1/(4 sigma^2)) ~ 0.94
    c = np.mean(np.sum(q[:-1] * q[1:], axis=1)) / 64
    assert c > 0.7


def test_query_mean_offset():
    """q_mean shifts every query of a head by the same vector 30 (1 + 0.5 z),
    leaving K, V and the spread of Q unchanged."""
    w0 = synth.get("bidir5").with_(name="x", H=1, grid=(2, 6, 8))
    w1 = w0.with_(q_mean=30.0)
    q0, k0, v0 = synth.head_base(w0, 0, 0)
    q1, k1, v1 = synth.head_base(w1, 0, 0)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    shift = q1 - q0
    assert np.allclose(shift, shift[0][None, :], atol=1e-9)
    assert 20.0 < shift[0].mean() < 40.0 and shift[0].std() > 5.0
    assert np.allclose(q1.std(axis=0), q0.std(axis=0), atol=1e-9)
