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


FILL = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>, std::array<char*, 1ul> >(int)"
SPARSE = "void mcs::(anonymous namespace)::sparse_ring_kernel<128, 64, true>(mcs::(anonymous namespace)::Params)"
SPARSE_SHORT = "sparse_ring_kernel<128, 64, true>"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, rows):
    """A rocprofv3 counter-collection CSV with the columns the summaries read."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for i, (kernel, counter, value, dur_ns) in enumerate(rows, 1):
            w.writerow([i, kernel, counter, value, 1000 * i, 1000 * i + dur_ns])


def test_traffic_summary_scales_by_the_copy_and_keeps_timed_launches(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE in KiB per dispatch, scaled so that the 1 GiB
    copy reads 1 GiB; traffic.json takes the timed (post-flush) launches."""
    sys.path.insert(0, ROOT)
    import bench
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "hash-" + k)
    gib_kib = float(1 << 20)
    fetch = [(COPY, "FETCH_SIZE", gib_kib / 2, 1), (FILL, "FETCH_SIZE", 0.0, 1), (SPARSE, "FETCH_SIZE", 1000.0, 1),
             (SPARSE, "FETCH_SIZE", 10.0, 1)]            # second sparse launch: not after the fill
    write = [(COPY, "WRITE_SIZE", gib_kib, 1), (FILL, "WRITE_SIZE", 5.0, 1), (SPARSE, "WRITE_SIZE", 100.0, 1),
             (SPARSE, "WRITE_SIZE", 1.0, 1)]
    _counter_csv(tmp_path / "f.csv", fetch)
    _counter_csv(tmp_path / "w.csv", write)
    bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cfg", "cmd-f", "cmd-w")
    import json
    t = json.load(open(tmp_path / "profiles" / "traffic.json"))[SPARSE_SHORT]["cfg"]
    assert t["fetch_factor"] == 2.0 and t["write_factor"] == 1.0 and t["launches"] == 1
    assert t["fetch_bytes"] == round(1000.0 * 1024 * 2) and t["write_bytes"] == round(100.0 * 1024)
    assert t["source_hash"] == "hash-sparse_ring_kernel"
    md = open(tmp_path / "profiles" / "traffic_cfg.md").read()
    assert "cmd-f" in md and "(untimed: warm-cache or fidelity call)" in md


def test_counter_summary_writes_the_cycle_columns(tmp_path, monkeypatch):
    """GRBM_GUI_ACTIVE per dispatch becomes cycles per launch and cycles per
    ns of the dispatch's own duration; columns of absent counters are left
    out."""
    sys.path.insert(0, ROOT)
    import bench
    rows = [(FILL, "GRBM_GUI_ACTIVE", 2e3, 100), (SPARSE, "GRBM_GUI_ACTIVE", 8e6, 500000)]
    _counter_csv(tmp_path / "c.csv", rows)
    out = tmp_path / "clock.md"
    monkeypatch.setattr(bench, "CLOCK_FILE", str(tmp_path / "clock.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "hash-" + k)
    bench.summarize_pmc(str(out), [(str(tmp_path / "c.csv"), "the command")], "T", "N")
    import json
    c = json.load(open(tmp_path / "clock.json"))[SPARSE_SHORT]["bidir5"]
    assert c["mhz"] == 2000.0 and c["source_hash"] == "hash-sparse_ring_kernel"  # 16 cycles/ns over 8 XCDs
    md = open(out).read()
    assert "GRBM_GUI_ACTIVE (M cycles)" in md and "MFMA busy %" not in md
    row = [l for l in md.splitlines() if l.startswith("| `sparse_ring_kernel<128, 64, true>`")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert cells[1] == "1" and cells[2] == "500.0" and cells[3] == "8.00" and cells[4] == "16.000"
