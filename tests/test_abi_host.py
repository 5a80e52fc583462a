"""Host-side checks of the C ABI (not gpu): the library loads, exports every
symbol the header declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

from sparse_attention_video_pddp_amd import mcs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "mcs.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mcs_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mcs.lib()
    names = declared_functions()
    assert set(names) == set(mcs.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    assert L.mcs_version() >= 100


def test_status_strings():
    L = mcs.lib()
    for code, name in enumerate(["MCS_OK", "MCS_ERR_INVALID_ARG", "MCS_ERR_UNSUPPORTED", "MCS_ERR_WORKSPACE",
                                 "MCS_ERR_HIP"]):
        assert L.mcs_status_string(code).decode() == name


def base(**kw):
    d = dict(B=1, H=2, Nq=1000, Nkv=1200, d=128, group_size=64, k=60, scale=None, causal_block=0,
             q_offset=0, pddp_iters=32, dtype="bf16")
    d.update(kw)
    return mcs.problem(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), mcs.MCS_ERR_UNSUPPORTED),
    (dict(group_size=32), mcs.MCS_ERR_UNSUPPORTED),
    (dict(k=0), mcs.MCS_ERR_INVALID_ARG),
    (dict(k=1201), mcs.MCS_ERR_INVALID_ARG),
    (dict(Nkv=0, k=1), mcs.MCS_ERR_INVALID_ARG),
    (dict(Nq=-1), mcs.MCS_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mcs.MCS_ERR_INVALID_ARG),
    (dict(scale=0.0), mcs.MCS_ERR_INVALID_ARG),
    (dict(causal_block=-3), mcs.MCS_ERR_INVALID_ARG),
    (dict(q_offset=-1), mcs.MCS_ERR_INVALID_ARG),
    (dict(pddp_iters=5000), mcs.MCS_ERR_INVALID_ARG),
    (dict(B=300, H=300), mcs.MCS_ERR_UNSUPPORTED),
    (dict(Nkv=1 << 22, k=60), mcs.MCS_ERR_UNSUPPORTED),   # one head's K > 2^31 bytes (32-bit offsets)
    (dict(dtype="f32", r_dtype="bf16"), mcs.MCS_ERR_UNSUPPORTED),  # a bf16 residual needs bf16 inputs
])
def test_bad_problem_is_rejected_before_launch(kw, code):
    p = base(**kw)
    with pytest.raises(mcs.MCSError) as e:
        mcs.dense_attn(p, 16, 16, 16, 32, None, stream=0)
    assert e.value.status == code
    b = ctypes.c_size_t()
    assert mcs.lib().mcs_workspace_size(ctypes.byref(p), 0, ctypes.byref(b), None) == code


def test_bad_dtype_rejected():
    p = base()
    p.dtype = 7
    with pytest.raises(mcs.MCSError) as e:
        mcs.sparse_attn(p, 16, 16, 16, 16, 16, None, 32, stream=0)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED
    p = base()
    p.r_dtype = 5
    with pytest.raises(mcs.MCSError) as e:
        mcs.sparse_attn(p, 16, 16, 16, 16, 16, None, 32, stream=0)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED and "r_dtype" in str(e.value)


def test_anchor_mode_field():
    """anchor_mode: 0 (automatic) by default; an unknown value is refused;
    the single pass needs bf16 inputs and at most 32768 visible keys; it needs
    no mass matrix, so its anchor workspace is smaller."""
    assert base().anchor_mode == mcs.MCS_ANCHOR_AUTO == 0
    p = base()
    p.anchor_mode = 3
    with pytest.raises(mcs.MCSError) as e:
        mcs.workspace_size(p, mcs.MCS_WS_ANCHOR)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "anchor_mode" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:
        mcs.workspace_size(base(dtype="f32", anchor_mode="single_pass"), mcs.MCS_WS_ANCHOR)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED
    with pytest.raises(mcs.MCSError) as e:
        mcs.workspace_size(base(Nkv=40000, k=60, anchor_mode="single_pass"), mcs.MCS_WS_ANCHOR)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED
    two = mcs.workspace_size(base(anchor_mode="two_pass"), mcs.MCS_WS_ANCHOR)
    one = mcs.workspace_size(base(anchor_mode="single_pass"), mcs.MCS_WS_ANCHOR)
    c = -(-1000 // 64)
    assert one[0] == one[1] and two[1] - one[1] >= 4 * c * 1200 and two[0] - one[0] >= 2 * 4 * c * 1200
    # a causal query chunk whose queries see only the first 2 of 10 frames of a long cache
    causal = base(Nq=256, Nkv=64 * 1024, k=600, causal_block=1024, q_offset=1024, anchor_mode="single_pass")
    mcs.workspace_size(causal, mcs.MCS_WS_ANCHOR)


def test_residual_dtype_defaults_to_float32():
    """A problem with r_dtype left at zero keeps R in float32; every kept-key
    count up to Nkv is accepted (no on-chip table limits k)."""
    p = base()
    assert p.r_dtype == mcs.MCS_F32 == 0
    assert base(r_dtype="bf16").r_dtype == mcs.MCS_BF16
    for k in (1, 28673, 40000):
        mcs.workspace_size(base(Nkv=40000, k=k), mcs.MCS_WS_ANCHOR)
    assert ctypes.sizeof(mcs.Problem) == 14 * 4


def test_null_and_misaligned_pointers_rejected():
    p = base()
    with pytest.raises(mcs.MCSError) as e:
        mcs.dense_attn(p, None, 16, 16, 32, None, stream=0)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "Q is NULL" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:
        mcs.sparse_attn(p, 16, 16, 16, 16, 16 + 4, None, 32, stream=0)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "idx" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:
        mcs.anchor(p, 16, 16, 16, 16, 32, 48, None, 64, ws_bytes=1 << 30, stream=0)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "R is NULL" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:
        mcs.group(p, 16, None, 64, ws_bytes=1 << 30, stream=0)
    assert "perm is NULL" in str(e.value)


def test_empty_problem_is_a_noop_without_pointers():
    p = base(Nq=0)
    mcs.dense_attn(p, None, None, None, None, None, stream=0)
    mcs.sparse_attn(p, None, None, None, None, None, None, None, stream=0)
    assert mcs.workspace_size(p, mcs.MCS_WS_ANCHOR) == (0, 0)
    p = base(H=0)
    mcs.group(p, None, None, None, ws_bytes=0, stream=0)


def test_workspace_sizes():
    p = base(anchor_mode="two_pass")
    g, gmin = mcs.workspace_size(p, mcs.MCS_WS_GROUP)
    assert g == gmin and g >= 2 * 4 * 2 * 1000
    a, amin = mcs.workspace_size(p, mcs.MCS_WS_ANCHOR)
    c = -(-1000 // 64)
    assert amin >= 4 * 2 * 1000 + 4 * c * 1200
    assert a >= amin + 4 * c * 1200
    # bf16: the anchor also keeps the float32 dense output of every head (2 heads x 1000 x 128)
    a32, amin32 = mcs.workspace_size(base(dtype="f32", anchor_mode="two_pass"), mcs.MCS_WS_ANCHOR)
    assert amin - amin32 >= 4 * 2 * 1000 * 128 and a - a32 == amin - amin32
    with pytest.raises(mcs.MCSError) as e:
        mcs.workspace_size(p, 9)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG


def test_block_select_workspace_and_limits():
    p = base()
    b, bmin = mcs.workspace_size(p, mcs.MCS_WS_BLOCK)
    # float32 pooled vectors: 16 query tiles and 19 key tiles of 2 heads
    assert b == bmin == 4 * 2 * (16 + 19) * 128
    with pytest.raises(mcs.MCSError) as e:      # workspace too small
        mcs.block_select(p, 16, 16, 32, 48, 64, ws_bytes=b - 1, stream=0)
    assert e.value.status == mcs.MCS_ERR_WORKSPACE
    with pytest.raises(mcs.MCSError) as e:
        mcs.block_select(p, 16, 16, None, 48, 64, ws_bytes=b, stream=0)
    assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "perm is NULL" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:      # 8193 KV blocks
        mcs.block_select(base(Nkv=8193 * 64, k=10, d=64), 16, 16, 32, 48, 64, ws_bytes=1 << 40, stream=0)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED
    with pytest.raises(mcs.MCSError) as e:      # 513 blocks to rank (float32: no kept-key table limit)
        mcs.block_select(base(Nkv=40000, k=32706, dtype="f32"), 16, 16, 32, 48, 64, ws_bytes=1 << 40, stream=0)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED
    mcs.block_select(base(Nq=0), None, None, None, None, None, ws_bytes=0, stream=0)


def test_residual_drift_workspace_and_limits():
    p = base()
    b, bmin = mcs.workspace_size(p, mcs.MCS_WS_DRIFT)
    assert b == bmin > 0
    for n in (0, 129):
        with pytest.raises(mcs.MCSError) as e:
            mcs.residual_drift(p, 16, 16, 16, 16, 16, 32, 48, n_rows=n, ws_bytes=b, stream=0)
        assert e.value.status == mcs.MCS_ERR_INVALID_ARG and "n_rows" in str(e.value)
    with pytest.raises(mcs.MCSError) as e:      # the workspace size is for the largest n_rows
        mcs.residual_drift(p, 16, 16, 16, 16, 16, 32, 48, n_rows=128, ws_bytes=b - 1, stream=0)
    assert e.value.status == mcs.MCS_ERR_WORKSPACE
    with pytest.raises(mcs.MCSError) as e:      # fewer rows need less: 8/128 of it is not enough for 9
        mcs.residual_drift(p, 16, 16, 16, 16, 16, 32, 48, n_rows=9, ws_bytes=b * 8 // 128, stream=0)
    assert e.value.status == mcs.MCS_ERR_WORKSPACE
    mcs.residual_drift(base(Nq=0), None, None, None, None, None, None, None, n_rows=8, ws_bytes=0, stream=0)


def test_noalloc_drift_limits_on_the_host():
    """The allocation-free check refuses, before touching any device, a
    problem whose scratch exceeds its 64 MiB static array, and bad row counts;
    an empty problem is a no-op."""
    big = mcs.problem(1, 40, 75600, 75600, 128, 128, 2268, dtype="bf16")
    with pytest.raises(mcs.MCSError) as e:
        mcs.residual_drift_noalloc(big, 16, 16, 16, 16, 16, 32, n_rows=128, stream=0)
    assert e.value.status == mcs.MCS_ERR_WORKSPACE and "static scratch" in str(e.value)
    for n in (0, 129):
        with pytest.raises(mcs.MCSError) as e:
            mcs.residual_drift_noalloc(base(), 16, 16, 16, 16, 16, 32, n_rows=n, stream=0)
        assert e.value.status == mcs.MCS_ERR_INVALID_ARG
    mcs.residual_drift_noalloc(base(Nq=0), None, None, None, None, None, None, n_rows=8, stream=0)


def test_drift_rows_are_spread_and_bounded():
    assert mcs.drift_rows(32760, 64)[0] >= 0 and mcs.drift_rows(32760, 64)[-1] < 32760
    assert len(mcs.drift_rows(32760, 64)) == 64 and len(mcs.drift_rows(32760, 500)) == 128
    assert mcs.drift_rows(5, 64) == [0, 1, 2, 3, 4]
    r = mcs.drift_rows(1000, 10)
    assert all(b - a == 100 for a, b in zip(r, r[1:]))


def test_adaptive_schedule_decisions():
    d = mcs.AdaptiveAnchoring.decide
    assert not d(0.01, 0.02, 1, 0) and d(0.03, 0.02, 1, 0)
    assert d(0.0, 0.02, 4, 5) and not d(0.0, 0.02, 3, 5)   # max_period counts steps since the anchor
    assert d(float("nan"), 0.02, 1, 0)                     # a broken measurement anchors
