"""bench.py's command-line contract on the host (not gpu): it measures one
GPU only, so more than one GPU, asked for by flag or by a distributed
launcher's environment, ends with a message and status 2 before anything
touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_help_lists_the_contract_flags():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--config"):
        assert flag in r.stdout


def test_launch_labels_follow_the_previous_kernel():
    """Profile rows: a launch right after the cache-flush fill is a timed call
    (plain name); the gathered-attention and dense kernels' other launches get
    rows of their own."""
    sys.path.insert(0, ROOT)
    import bench
    fill = "at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>, std::array<char*, 1ul> >"
    sp, dn = "sparse_ring_kernel<128, 64>", "dense_bf16_kernel<128, 8>"
    assert bench.launch_label(sp, fill) == sp
    assert bench.launch_label(sp, "topk_kernel<512, 64>") == sp + " (anchor epilogue)"
    assert bench.launch_label(sp, "block_select_sort_kernel<128>") == sp + " (block-sparse comparator)"
    assert bench.launch_label(sp, sp).endswith("(untimed: warm-cache or fidelity call)")
    assert bench.launch_label(dn, fill) == dn
    assert bench.launch_label(dn, "pddp_small_kernel<128>") == dn + " (anchor)"
    assert bench.launch_label(dn, dn) == dn + " (untimed)"
    assert bench.launch_label("mass_bf16_kernel<128, 64, 4>", dn) == "mass_bf16_kernel<128, 64, 4>"
