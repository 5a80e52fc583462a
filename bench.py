"""Benchmark of the MC-Sparse hot path on one MI355X.

One bench step is one anchor period of the denoising schedule over the whole
hot path: PDDP grouping + anchor (exact dense attention, per-group column
mass, top-k, anchor sparse attention and residual) on the anchor step's
inputs, then the reuse steps (gathered sparse attention + R) on the following
steps' drifted inputs.  All inputs are generated up front and resident in HBM
before the timed region.  Every library call is bracketed by HIP events on
the stream the library launches on; the metric is the reuse step
(mcs_sparse_attn).  The library's own exact attention (mcs_dense_attn) is
timed on the same rotating inputs as the comparator, and so is the
block-sparse comparator at the same token budget (mean-pooled block selection
from each step's Q/K, mcs_block_select, then mcs_sparse_attn without a
residual), and the residual-drift check of adaptive anchoring
(mcs_residual_drift, 64 sampled rows per head).  Before every timed call
a 512 MB scratch buffer (twice the 256 MB Infinity Cache) is overwritten, so
headline times are cold-cache; warm-cache times (back-to-back calls on one
step's inputs) are reported beside them.

Prints one JSON line (rank 0).  See --help.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/call + effective TFLOP/s (% bf16 MFMA peak) of sparse reuse step, N=32760"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed anchor periods")
    ap.add_argument("--warmup", type=int, default=2, help="untimed anchor periods")
    ap.add_argument("--config", default="bidir5", help="workload name (synth.CONFIGS)")
    ap.add_argument("--cpu-heads", type=int, default=1, help="heads in the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not overwrite the cache-flush buffer between calls")
    ap.add_argument("--no-fidelity", action="store_true",
                    help="skip the untimed fidelity diagnostic (reuse output against exact attention)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm-cache reuse calls (profiler counter runs: every reuse launch is then cold)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for profiler counter calibration)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DB", "OUT_MD", "CMD"),
                    help="write a markdown kernel table from a rocprofv3 kernel-trace database and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CMD_FETCH", "CMD_WRITE"),
                    help="derive per-launch HBM traffic from FETCH_SIZE/WRITE_SIZE counter CSVs of --config, "
                         "update profiles/traffic.json and exit")
    ap.add_argument("--stream", action="store_true",
                    help="instead of the metric: chunked-causal streaming of the frame-causal workload's whole "
                         "video (chunks of its query-chunk length, each an anchor and reuse steps over the "
                         "K/V cache); prints one JSON line of per-chunk times")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="OUT_MD then pairs CSV CMD of rocprofv3 derived-counter runs (MfmaUtil, MfmaFlopsBF16, "
                         "LdsUtil, LdsBankConflict, VALUBusy): write a per-kernel markdown table and exit")
    ap.add_argument("--title", default="", help="title for --summarize-trace")
    ap.add_argument("--note", default="", help="paragraph for --summarize-trace")
    return ap.parse_args()


# Kernels whose HBM traffic is reported, and the sources that define them:
# a stored counter reading is used only while these files are unchanged.
KERNEL_SOURCES = {
    "sparse_ring_kernel": ("sparse_bf16.hip", "ring.hpp", "mcs_device.hpp"),
    "dense_bf16_kernel": ("attn_bf16.hip", "mcs_device.hpp"),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_attention_video_pddp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, config: str):
    """HBM bytes per launch of a kernel instantiation (full name, e.g.
    "sparse_ring_kernel<128, 64, true>") measured with rocprofv3 counters, if
    they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel, {}).get(config)
    if not e or e.get("source_hash") != kernel_source_hash(kernel.split("<")[0]):
        return None
    return e.get("bytes_per_launch")


CLOCK_FILE = os.path.join(ROOT, "profiles", "clock.json")
N_XCD = 8  # GRBM_GUI_ACTIVE is summed over the chip's XCDs
N_CU = 256  # texture units (one address and one data unit per CU) summed by the _sum counters


def load_clock(kernel: str, config: str):
    """Engine clock (MHz) during the kernel's timed launches, from
    GRBM_GUI_ACTIVE per ns of a counter run on the current kernel source;
    else None."""
    try:
        with open(CLOCK_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel, {}).get(config)
    if not e or e.get("source_hash") != kernel_source_hash(kernel.split("<")[0]):
        return None
    return e.get("mhz")


def _short_kernel(name: str) -> str:
    import re
    m = re.match(r"_ZN3mcs12_GLOBAL__N_1(\d+)", name)
    if m:  # names the profiler leaves mangled (a __bf16 template argument): name<args>
        n = int(m.group(1))
        rest = name[m.end():]
        ident, rest = rest[:n], rest[n:]
        pretty = []
        for a in re.finditer(r"DF16b|Li(\d+)E|Lb([01])E|(?<=I)f|(?<=E)f", rest.split("EEv")[0]):
            if a.group(0) == "DF16b":
                pretty.append("__bf16")
            elif a.group(1):
                pretty.append(a.group(1))
            elif a.group(2):
                pretty.append("true" if a.group(2) == "1" else "false")
            else:
                pretty.append("float")
        return ident + (f"<{', '.join(pretty)}>" if pretty else "")
    name = name.replace("void ", "").replace("mcs::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


FLUSH_KERNEL = "FillFunctor<unsigned char>"   # the 512 MB cache-flush fill before every timed call


def launch_label(kernel: str, prev: str) -> str:
    """Row of a launch in the profile summaries, from the kernel launched just
    before it.  Every timed call of the bench starts right after the cache
    flush, so a launch right after the flush fill is a timed (cold) call and
    keeps the plain kernel name: those rows are comparable with the live
    HIP-event timings.  The gathered-attention kernel otherwise is the anchor's
    epilogue (after a top-k or single-pass selection launch: it forms R), the
    block-sparse comparator
    (after a block selection) or an untimed call (warm-cache or fidelity
    pass); the dense kernel after a PDDP launch is the anchor's exact pass,
    else an untimed call."""
    cold = FLUSH_KERNEL in prev
    if kernel.startswith("sparse_ring_kernel"):
        if prev.startswith("topk_kernel") or prev.startswith("anchor_fused"):
            return kernel + " (anchor epilogue)"
        if prev.startswith("block_select"):
            return kernel + " (block-sparse comparator)"
        return kernel if cold else kernel + " (untimed: warm-cache or fidelity call)"
    if kernel.startswith("dense_bf16_kernel") or kernel.startswith("dense_f32_kernel"):
        if cold:
            return kernel
        return kernel + (" (anchor)" if prev.startswith("pddp") else " (untimed)")
    return kernel


def summarize_trace(db: str, out: str, title: str, cmd: str, note: str) -> None:
    """Markdown table of per-kernel durations from a rocprofv3 kernel-trace
    database (its `kernels` view, read with sqlite3).  Launches are split into
    rows by launch_label, so that the rows of timed calls are comparable with
    the live timings (reuse_ms_per_call, dense_ms_per_call)."""
    import sqlite3
    con = sqlite3.connect(os.path.abspath(db))
    rows = con.execute("select name, start, end from kernels order by start").fetchall()
    con.close()
    stats, prev = {}, ""
    for name, t0, t1 in rows:
        k = _short_kernel(name)
        stats.setdefault(launch_label(k, prev), []).append((t1 - t0) / 1e3)
        prev = k
    total = sum(sum(v) for v in stats.values())
    with open(out, "w") as f:
        f.write(f"# {title}\n\nCommand (repository root, one MI355X; `cd /tmp && export TMPDIR=/tmp` for the "
                f"profiler's scratch):\n\n```\n{cmd}\n```\n\n")
        if note:
            f.write(note + "\n\n")
        f.write("| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | % time |\n"
                "|---|---:|---:|---:|---:|---:|---:|\n")
        for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
            f.write(f"| `{k}` | {len(v)} | {statistics.fmean(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                    f"{sum(v) / 1e3:.2f} | {100 * sum(v) / total:.1f} |\n")
    print(open(out).read())


def summarize_counters(fetch_csv: str, write_csv: str, config: str, cmd_fetch: str, cmd_write: str) -> None:
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB
    device copy of the same run.  Launches are split into rows by
    launch_label; traffic.json holds the rows of timed (cold) calls, the ones
    the live timings measure.  Writes profiles/traffic.json and a markdown
    summary."""
    import csv
    per = {}
    for tag, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        vals, prev = {}, ""
        for r in rows:
            if r["Counter_Name"] != tag:
                continue
            k = _short_kernel(r["Kernel_Name"])
            vals.setdefault(launch_label(k, prev), []).append(float(r["Counter_Value"]))
            prev = k
        per[tag] = vals
    copy = [k for k in per["FETCH_SIZE"] if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no device copy in the counter runs (run bench.py with --copy-calibration)")
    gib_kib = float(1 << 20)

    def copy_reading(tag):
        # median over the 1 GiB copies (other, small device copies share the kernel name)
        v = per[tag][copy[0]]
        return statistics.median(x for x in v if x > 0.25 * max(v))

    f_read, w_read = copy_reading("FETCH_SIZE"), copy_reading("WRITE_SIZE")
    f_fac, w_fac = gib_kib / f_read, gib_kib / w_read
    try:
        with open(TRAFFIC_FILE) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    lines = [f"# HBM traffic per launch, {config}\n",
             "Two counter runs of the same command (repository root, one MI355X):\n",
             f"```\n{cmd_fetch}\n{cmd_write}\n```\n",
             f"Calibration: the 1 GiB device copies in the same runs read FETCH_SIZE = "
             f"{f_read:.0f} KiB and WRITE_SIZE = {w_read:.0f} KiB (median per copy), so fetch counts are "
             f"scaled by {f_fac:.3f} and write counts by {w_fac:.3f}.\n",
             "| kernel | launches | fetch (MB/launch) | write (MB/launch) | total (MB/launch) |",
             "|---|---:|---:|---:|---:|"]
    for k in sorted(per["FETCH_SIZE"]):
        if k not in per["WRITE_SIZE"] or "copyBuffer" in k:
            continue
        fb = statistics.fmean(per["FETCH_SIZE"][k]) * 1024 * f_fac
        wb = statistics.fmean(per["WRITE_SIZE"][k]) * 1024 * w_fac
        lines.append(f"| `{k}` | {len(per['FETCH_SIZE'][k])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                     f"{(fb + wb) / 1e6:.1f} |")
        base = k.split("<")[0]
        if base in KERNEL_SOURCES and "(" not in k:
            table.setdefault(k, {})[config] = {
                "bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
                "launches": len(per["FETCH_SIZE"][k]), "source_hash": kernel_source_hash(base)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    out = os.path.join(ROOT, "profiles", f"traffic_{config}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(out).read())


def summarize_pmc(out: str, runs, title: str, note: str) -> None:
    """Per-kernel means of rocprofv3 derived counters (one row per kernel
    label, launch_label), from one or more counter runs; MFMA TFLOP/s from
    MfmaFlopsBF16 over each dispatch's own duration (counter runs serialise
    the dispatches)."""
    import csv
    vals = {}
    for path, _ in runs:
        rows = sorted(csv.DictReader(open(path)), key=lambda r: (int(r["Dispatch_Id"]), r["Counter_Name"]))
        prev, last_id = "", None
        per = {}  # this run's counters of each dispatch, for ratios between counters of one dispatch
        for r in rows:
            k = _short_kernel(r["Kernel_Name"])
            if r["Dispatch_Id"] != last_id:
                label = launch_label(k, prev)
                prev, last_id = k, r["Dispatch_Id"]
            d = vals.setdefault(label, {})
            v = float(r["Counter_Value"])
            d.setdefault(r["Counter_Name"], []).append(v)
            per.setdefault((label, r["Dispatch_Id"]), {})[r["Counter_Name"]] = v
            dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            if r["Counter_Name"] == "MfmaFlopsBF16":
                d.setdefault("tflops", []).append(v / dt / 1e12 if dt > 0 else 0.0)
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                # GPU-busy cycles of the dispatch (summed over the XCDs) and their rate
                d.setdefault("mcycles", []).append(v / 1e6)
                d.setdefault("cyc_per_ns", []).append(v / (dt * 1e9) if dt > 0 else 0.0)
                d.setdefault("dur_us", []).append(dt * 1e6)
        for (label, _), c in per.items():
            d, gui = vals[label], c.get("GRBM_GUI_ACTIVE", 0.0)
            # busy cycles summed over the units of every CU, against the dispatch's cycles per XCD
            for name, key in (("TA_TA_BUSY_sum", "ta_busy"), ("TD_TD_BUSY_sum", "td_busy")):
                if name in c and gui > 0:
                    d.setdefault(key, []).append(100.0 * c[name] / N_CU / (gui / N_XCD))
            if "SQ_WAIT_ANY" in c and c.get("SQ_WAVE_CYCLES", 0.0) > 0:
                d.setdefault("wave_wait", []).append(100.0 * c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"])
    cols = [("MfmaUtil", "MFMA busy %", 1), ("tflops", "MFMA TFLOP/s", 1), ("LdsUtil", "LDS busy %", 1),
            ("LdsBankConflict", "bank-conflict cycles per LDS cycle", 3), ("VALUBusy", "VALU busy %", 1),
            ("dur_us", "duration (us)", 1), ("mcycles", "GRBM_GUI_ACTIVE (M cycles)", 2),
            ("cyc_per_ns", "GRBM_GUI_ACTIVE per ns", 3), ("wave_wait", "waves waiting %", 1),
            ("ta_busy", "texture address busy %", 1), ("td_busy", "texture data busy %", 1)]
    cols = [c for c in cols if any(c[0] in d for d in vals.values())]  # only counters of these runs
    config = os.environ.get("MCS_BENCH_CONFIG", "bidir5")
    clock = {}
    for k, d in vals.items():
        base = k.split("<")[0]
        if "cyc_per_ns" in d and base in KERNEL_SOURCES and "(" not in k:  # timed launches only
            clock.setdefault(k, {})[config] = {
                "mhz": round(statistics.fmean(d["cyc_per_ns"]) / N_XCD * 1e3, 1),
                "launches": len(d["cyc_per_ns"]), "source_hash": kernel_source_hash(base)}
    if clock:
        try:
            with open(CLOCK_FILE) as fh:
                table = json.load(fh)
        except (OSError, ValueError):
            table = {}
        for k, e in clock.items():
            table.setdefault(k, {}).update(e)
        with open(CLOCK_FILE, "w") as fh:
            json.dump(table, fh, indent=1, sort_keys=True)
    with open(out, "w") as f:
        f.write(f"# {title}\n\nCommands (repository root, one MI355X; one run per counter set):\n\n```\n")
        for _, cmd in runs:
            f.write(cmd + "\n")
        f.write("```\n\n")
        if note:
            f.write(note + "\n\n")
        f.write("| kernel | launches | " + " | ".join(c[1] for c in cols) + " |\n|---|---:|" +
                "---:|" * len(cols) + "\n")
        order = "MfmaUtil" if any("MfmaUtil" in d for d in vals.values()) else "dur_us"
        for k in sorted(vals, key=lambda k: -statistics.fmean(vals[k].get(order, [0.0]))):
            d = vals[k]
            n = max(len(v) for v in d.values())
            cells = [f"{statistics.fmean(d[c]):.{nd}f}" if c in d else "" for c, _, nd in cols]
            f.write(f"| `{k}` | {n} | " + " | ".join(cells) + " |\n")
    print(open(out).read())


def device_max_sclk_mhz() -> float:
    """Maximum engine clock of the first gfx950 agent, from rocminfo (run as
    a child process); 0 when it cannot be read."""
    import subprocess
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return 0.0
    gpu = False
    for line in out.splitlines():
        if "gfx950" in line:
            gpu = True
        if gpu and "Max Clock Freq. (MHz)" in line:
            try:
                return float(line.split(":")[1].split()[0])
            except (IndexError, ValueError):
                return 0.0
    return 0.0


def reuse_bytes_per_launch(w) -> float:
    """Logical bytes of one mcs_sparse_attn call: per (b,h,group) the k
    gathered K and V rows and the group's Q and O rows (input dtype), its R
    rows (float32) and the k indices (int32)."""
    e = 2 if w.dtype == "bf16" else 4
    BH = w.B * w.H
    return BH * (w.n_groups * (2 * w.k * w.d * e + 4 * w.k) + w.Nq * w.d * (2 * e + 4))


def dense_flops(w) -> float:
    """4*d per visible (query, key) pair (QK^T and PV)."""
    if w.causal_block == 0:
        pairs = w.Nq * w.Nkv
    else:
        pairs = 0
        for i in range(w.Nq):
            pairs += min(w.Nkv, ((w.q_offset + i) // w.causal_block + 1) * w.causal_block)
    return 4.0 * w.d * pairs * w.B * w.H


def reuse_flops(w) -> float:
    return 4.0 * w.d * w.Nq * w.k * w.B * w.H


def workload_kind(w) -> str:
    """The attention pattern and sizes of a workload, in words."""
    t, y, x = w.grid
    gen = "Fourier-feature Q/K" if w.generator == "fourier" else "smoothed-random-field Q/K"
    if w.causal_block and w.q_frames is not None:
        t0, t1 = w.q_frames
        return (f"frame-block-causal attention of a {t1 - t0}-frame query chunk (frames {t0}..{t1 - 1}, "
                f"{w.Nq} tokens) over a {t}x{y}x{x} = {w.Nkv}-token K/V cache, {gen}")
    return f"full bidirectional 3D attention over a {t}x{y}x{x} = {w.Nkv}-token video latent, {gen}"


def cpu_baseline(w, host0, host1, nheads: int, reuse_budget_s: float = 10.0):
    """The oracle as it stands, on a bounded sample: its own anchor (PDDP,
    dense attention, column mass, top-k, residual) prepares each sampled
    head, then its reuse step (the metric's operation) is timed, repeated
    until about reuse_budget_s seconds per head are timed, and its dense
    attention (the comparator) once on the same step-1 inputs.  The value is
    in the metric's unit: executed FLOPs of the reuse step per second."""
    import numpy as np
    from oracle.mcs_oracle import anchor_step, dense_attention, reuse_step
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    heads = sorted(host0)[:nheads]
    t_anchor = t_reuse = t_dense = 0.0
    runs = 0  # head reuse steps timed
    for bh in heads:
        q0, k0, v0 = (x.astype(np.float64) for x in host0[bh])
        q1, k1, v1 = (x.astype(np.float64) for x in host1[bh])
        t0 = time.perf_counter()
        a = anchor_step(q0, k0, v0, w.group_size, w.k, w.scale, w.causal_block, w.q_offset, w.pddp_iters)
        t_anchor += time.perf_counter() - t0
        t_head = 0.0
        while True:
            t1 = time.perf_counter()
            reuse_step(q1, k1, v1, a["perm"], a["idx"], a["R"], w.group_size, w.scale, w.causal_block, w.q_offset)
            t_head += time.perf_counter() - t1
            runs += 1
            if t_head >= reuse_budget_s:
                break
        t_reuse += t_head
        t1 = time.perf_counter()
        dense_attention(q1, k1, v1, w.scale, w.causal_block, w.q_offset)
        t_dense += time.perf_counter() - t1
    BH = w.B * w.H
    n = len(heads)
    per_run = t_reuse / runs
    return {"value": round(reuse_flops(w) / BH / per_run / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} of {BH} heads of {w.name}: the oracle's reuse step (numpy fp64 gathered sparse "
                      f"attention + R, on the oracle's own anchor of step 0) on step-1 inputs, run {runs} times, "
                      f"{t_reuse:.1f} s timed ({per_run * 1e3:.0f} ms per head step); its dense attention once per "
                      f"head on the same inputs ({t_dense / n * 1e3:.0f} ms per head), after {t_anchor:.1f} s of "
                      f"oracle anchor work; value = executed reuse FLOPs (4 Nq k d per head) per second",
            "reuse_ms_per_head": round(per_run * 1e3, 1),
            "dense_ms_per_head": round(t_dense / n * 1e3, 1),
            "reuse_ms_per_call_extrapolated": round(per_run * BH * 1e3, 1),
            "dense_ms_per_call_extrapolated": round(t_dense / n * BH * 1e3, 1),
            "anchor_ms_per_call_extrapolated": round(t_anchor / n * BH * 1e3, 1),
            "cpu": platform.processor() or platform.machine(), "numpy": np.__version__}


def stream_main(args) -> None:
    """Chunked-causal streaming at full size: the frame-causal workload's video
    (grid T x H x W, chunks of its query-chunk length) generated chunk by chunk
    over a zero-initialised K/V cache of the whole video, once with each
    anchor mode (two-pass: column-mass matrix then top-k; single-pass: each
    group's mass kept on chip and selected in the same workgroup; both give
    the same selections).  Inputs: the workload's generator for the whole
    video at step 0 (queries of every frame), then per step an extra drift of
    the current chunk's rows drawn on the device (seeded, the same for both
    modes).  Timed with HIP events per call, caches flushed."""
    import torch
    from sparse_attention_video_pddp_amd import mcs, synth
    from sparse_attention_video_pddp_amd.workload import device_inputs

    base = synth.get("causal")
    T, Hg, Wg = base.grid
    fpc = base.q_frames[1] - base.q_frames[0]
    full = base.with_(name="causal_video", q_frames=(0, T))
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    (Qa, Ka, Va), _ = device_inputs(full, 0)
    ft = Hg * Wg
    n_chunks = T // fpc
    A = base.anchor_every
    steps = max(A, 4)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run(mode):
        mk = lambda: mcs.ChunkedCausalStream(full.B, full.H, full.d, ft, fpc, n_chunks, full.group_size,  # noqa
                                             full.k, full.scale, full.dtype, full.pddp_iters, anchor_mode=mode)
        # untimed: one anchor and one reuse step of a first chunk (first launches of every kernel)
        warm = mk()
        warm.begin_chunk()
        wr = warm.rows()
        for anchor in (True, False):
            warm.step(Qa[:, :, wr], Ka[:, :, wr], Va[:, :, wr], anchor)
        torch.cuda.synchronize()
        del warm
        st = mk()
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        rec = []
        for c in range(n_chunks):
            st.begin_chunk()
            r = st.rows()
            Q, K, V = Qa[:, :, r].clone(), Ka[:, :, r].clone(), Va[:, :, r].clone()
            for s in range(steps):
                if s:
                    for X in (Q, K, V):
                        X += (full.drift * torch.randn(X.shape, generator=gen, device=dev)).to(X.dtype)
                anchor = s % A == 0
                scratch.fill_(s & 255)
                a, b = ev(), ev()
                a.record(stream)
                st.step(Q, K, V, anchor, stream=stream)
                b.record(stream)
                rec.append((c, anchor, a, b))
        torch.cuda.synchronize()
        per = {}
        for c, anchor, a, b in rec:
            per.setdefault(c, {"anchor_ms": [], "reuse_ms": []})["anchor_ms" if anchor else "reuse_ms"].append(
                a.elapsed_time(b))
        total = sum(a.elapsed_time(b) for _, _, a, b in rec)
        return per, total, st.chunk_tokens, st.capacity

    res = {m: run(m) for m in ("auto", "two_pass", "single_pass")}
    per, total, chunk_tokens, capacity = res["auto"]
    chunks = []
    for c, v in sorted(per.items()):
        chunks.append({"chunk": c, "visible_keys": (c + 1) * chunk_tokens,
                       "anchor_ms": round(statistics.fmean(v["anchor_ms"]), 4),
                       "anchor_ms_two_pass": round(statistics.fmean(res["two_pass"][0][c]["anchor_ms"]), 4),
                       "anchor_ms_single_pass": round(statistics.fmean(res["single_pass"][0][c]["anchor_ms"]), 4),
                       "reuse_ms": round(statistics.fmean(v["reuse_ms"]), 4)})
    out = {"metric": "chunked-causal streaming: ms per chunk (group + anchor + reuse steps)",
           "value": round(total / n_chunks, 4), "unit": "ms", "higher_is_better": False, "n_gpus": 1,
           "dtype": full.dtype, "data": "synthetic",
           "config": {"workload": f"frame-causal video {T}x{Hg}x{Wg} = {T * ft} tokens, B={full.B}, H={full.H}, "
                                  f"d={full.d}, chunks of {fpc} frames ({chunk_tokens} queries), K/V cache "
                                  f"of {capacity} rows, groups of {full.group_size}, k={full.k}, {steps} steps "
                                  f"per chunk, anchor every {A}, residual R in float32",
                      "chunks": n_chunks, "steps_per_chunk": steps},
           "value_two_pass": round(res["two_pass"][1] / n_chunks, 4),
           "value_single_pass": round(res["single_pass"][1] / n_chunks, 4),
           "chunks": chunks, "anchor_ms_is": "mcs_group + mcs_anchor on the chunk's anchor step",
           "cache": "flushed (512 MB overwrite before every timed call)",
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        db, out, cmd = args.summarize_trace
        summarize_trace(db, out, args.title or f"Kernel trace, {args.config}", cmd, args.note)
        return
    if args.summarize_pmc:
        a = args.summarize_pmc
        if len(a) < 3 or len(a) % 2 == 0:
            raise SystemExit("--summarize-pmc OUT_MD CSV CMD [CSV CMD ...]")
        summarize_pmc(a[0], list(zip(a[1::2], a[2::2])), args.title or "Counters", args.note)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters[:2], args.config, *args.summarize_counters[2:])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every box here has one MI355X and the method's "
              "kernels run on one GPU's share; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if args.stream:
        stream_main(args)
        return
    import numpy as np
    import torch
    from sparse_attention_video_pddp_amd import mcs, synth
    from sparse_attention_video_pddp_amd.workload import device_inputs

    w = synth.get(args.config)
    p = mcs.problem_for(w)
    A = min(w.anchor_every, w.steps)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print(f"[bench] {w.name}: {p}", file=sys.stderr, flush=True)
    keep = [(0, h) for h in range(min(args.cpu_heads, w.H))] if not args.no_cpu_baseline else []
    step_in, host = [], {}
    for s in range(A):
        (Q, K, V), hs = device_inputs(w, s, keep_heads=keep)
        step_in.append((Q, K, V))
        host[s] = hs
    print(f"[bench] inputs resident: {A} steps x {3 * Q.numel() * Q.element_size() / 1e9:.2f} GB",
          file=sys.stderr, flush=True)
    st = mcs.MCSparseAttention(p)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    nflush = [0]

    def flush():
        # overwrite more than the Infinity Cache holds, outside every timed bracket
        if not args.no_flush:
            nflush[0] += 1
            scratch.fill_(nflush[0] & 255)

    def period(record):
        e0, e1, e2 = ev(), ev(), ev()
        flush()
        e0.record(stream)
        mcs.group(p, step_in[0][0], st.perm, st.ws_group, stream=stream)
        e1.record(stream)
        mcs.anchor(p, *step_in[0], st.perm, st.O, st.idx, st.R, st.ws_anchor, stream=stream)
        e2.record(stream)
        re = []
        for s in range(1, A):
            a, b = ev(), ev()
            flush()
            a.record(stream)
            mcs.sparse_attn(p, *step_in[s], st.perm, st.idx, st.R, st.O, stream=stream)
            b.record(stream)
            re.append((a, b))
        if record is not None:
            record.append(((e0, e1), (e1, e2), re))

    for _ in range(args.warmup):
        period(None)
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        period(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    group_ms = [a.elapsed_time(b) for (a, b), _, _ in rec]
    anchor_ms = [a.elapsed_time(b) for _, (a, b), _ in rec]
    reuse_ms = [a.elapsed_time(b) for _, _, re in rec for (a, b) in re]

    # comparator: the library's exact attention, same rotating inputs and count
    Od = torch.empty_like(st.O)
    for s in range(1, A):
        mcs.dense_attn(p, *step_in[s], Od, stream=stream)
    torch.cuda.synchronize()
    dense_ms = []
    for i in range(max(1, len(reuse_ms) // 2)):
        s = 1 + i % (A - 1)
        a, b = ev(), ev()
        flush()
        a.record(stream)
        mcs.dense_attn(p, *step_in[s], Od, stream=stream)
        b.record(stream)
        dense_ms.append((a, b))
    torch.cuda.synchronize()
    dense_ms = [a.elapsed_time(b) for a, b in dense_ms]

    # the reuse step with the residual stored in bf16 (r_dtype MCS_BF16, opt-in):
    # its own anchor (untimed), then the same cold protocol and count
    p16 = mcs.problem_for(w, "bf16") if w.dtype == "bf16" else None
    r16_ms = []
    if p16 is not None:
        st16 = mcs.MCSparseAttention(p16)
        st16.step(*step_in[0], True, stream=stream)
        torch.cuda.synchronize()
        r16_ev = []
        for i in range(max(1, len(reuse_ms) // 2)):
            s = 1 + i % (A - 1)
            a, b = ev(), ev()
            flush()
            a.record(stream)
            mcs.sparse_attn(p16, *step_in[s], st16.perm, st16.idx, st16.R, st16.O, stream=stream)
            b.record(stream)
            r16_ev.append((a, b))
        torch.cuda.synchronize()
        r16_ms = [a.elapsed_time(b) for a, b in r16_ev]
        del st16

    # the single-pass anchor (group masses on chip, selection in the same
    # workgroup) on the anchor step, same cold protocol, when the workload's rows fit
    sp_ms = []
    try:
        p1 = mcs.problem_for(w, anchor_mode="single_pass")
        mcs.workspace_size(p1, mcs.MCS_WS_ANCHOR)
    except mcs.MCSError:
        p1 = None
    if p1 is not None:
        st1 = mcs.MCSparseAttention(p1)
        mcs.group(p1, step_in[0][0], st1.perm, st1.ws_group, stream=stream)
        mcs.anchor(p1, *step_in[0], st1.perm, st1.O, st1.idx, st1.R, st1.ws_anchor, stream=stream)
        torch.cuda.synchronize()
        sp_ev = []
        for i in range(max(1, args.steps // 2)):
            # as in the timed periods: grouping right after the flush, the anchor after it
            a, b = ev(), ev()
            flush()
            mcs.group(p1, step_in[0][0], st1.perm, st1.ws_group, stream=stream)
            a.record(stream)
            mcs.anchor(p1, *step_in[0], st1.perm, st1.O, st1.idx, st1.R, st1.ws_anchor, stream=stream)
            b.record(stream)
            sp_ev.append((a, b))
        torch.cuda.synchronize()
        sp_ms = [a.elapsed_time(b) for a, b in sp_ev]
        del st1

    # block-sparse comparator at the same token budget: mean-pooled block
    # selection from the step's own Q/K, then the gathered attention (no residual)
    bsa = mcs.BlockSparseComparator(p)
    bsa.step(*step_in[1], stream=stream)
    torch.cuda.synchronize()
    bsa_ev = []
    for i in range(max(1, len(reuse_ms) // 2)):
        s = 1 + i % (A - 1)
        a, b, c = ev(), ev(), ev()
        flush()
        a.record(stream)
        mcs.block_select(p, step_in[s][0], step_in[s][1], bsa.perm, bsa.idx, bsa.ws, stream=stream)
        b.record(stream)
        mcs.sparse_attn(p, *step_in[s], bsa.perm, bsa.idx, None, bsa.O, stream=stream)
        c.record(stream)
        bsa_ev.append((a, b, c))
    torch.cuda.synchronize()
    bsel_ms = [a.elapsed_time(b) for a, b, _ in bsa_ev]
    bsa_ms = [a.elapsed_time(c) for a, _, c in bsa_ev]

    # residual-drift check of adaptive anchoring (64 sampled rows per head) on
    # a reuse output, same cold protocol
    drift_rows = torch.tensor(mcs.drift_rows(w.Nq, 64), dtype=torch.int32, device=dev)
    drift = torch.zeros(w.B * w.H + 1, dtype=torch.float32, device=dev)  # per head, then their maximum
    ws_drift = torch.empty(max(mcs.workspace_size(p, mcs.MCS_WS_DRIFT)[0], 1), dtype=torch.uint8, device=dev)
    mcs.residual_drift(p, *step_in[1], st.O, drift_rows, drift, ws_drift, stream=stream)
    torch.cuda.synchronize()
    drift_ev = []
    for i in range(max(1, len(reuse_ms) // 2)):
        s = 1 + i % (A - 1)
        a, b = ev(), ev()
        flush()
        a.record(stream)
        mcs.residual_drift(p, *step_in[s], st.O, drift_rows, drift, ws_drift, stream=stream)
        b.record(stream)
        drift_ev.append((a, b))
    torch.cuda.synchronize()
    drift_ms = [a.elapsed_time(b) for a, b in drift_ev]

    # fidelity diagnostic (untimed): relative error of the reuse output against the
    # library's exact attention on the same step, with and without the residual, by
    # steps since the anchor (the last timed period's anchor state is still in place)
    # Also: the block-sparse comparator recomputed on the step, and the exact
    # token selection recomputed on the step (an anchor on that step's inputs,
    # its sparse output without the residual): together they separate the
    # errors of block-granular pooled selection, of selection staleness and of
    # the discarded tail.
    fid_r, fid_nor, fid_stale, fid_bsa, fid_now, fid_drift = [], [], [], [], [], []
    if not args.no_fidelity:
        On = torch.empty_like(st.O)
        O0 = torch.empty_like(st.O)
        now = mcs.MCSparseAttention(p)
        mcs.dense_attn(p, *step_in[0], O0, stream=stream)  # the anchor step's exact output
        for s in range(1, A):
            mcs.dense_attn(p, *step_in[s], Od, stream=stream)
            ref = Od.float()
            nrm = ref.norm().item()
            rel = lambda O: round((O.float() - ref).norm().item() / nrm, 6)  # noqa: E731
            mcs.sparse_attn(p, *step_in[s], st.perm, st.idx, st.R, st.O, stream=stream)
            fid_r.append(rel(st.O))
            mcs.residual_drift(p, *step_in[s], st.O, drift_rows, drift, ws_drift, stream=stream)
            fid_drift.append(round(float(drift[-1].item()), 6))
            mcs.sparse_attn(p, *step_in[s], st.perm, st.idx, None, On, stream=stream)
            fid_nor.append(rel(On))
            fid_stale.append(rel(O0))
            fid_bsa.append(rel(bsa.step(*step_in[s], stream=stream)))
            now.step(*step_in[s], True, stream=stream)
            mcs.sparse_attn(p, *step_in[s], now.perm, now.idx, None, On, stream=stream)
            fid_now.append(rel(On))
        del On, O0, now
        torch.cuda.synchronize()

    # warm cache: back-to-back calls on one step's inputs, no flush
    warm = []
    for i in range(0 if args.no_warm else 23):
        a, b = ev(), ev()
        a.record(stream)
        mcs.sparse_attn(p, *step_in[1], st.perm, st.idx, st.R, st.O, stream=stream)
        b.record(stream)
        if i >= 3:
            warm.append((a, b))
    torch.cuda.synchronize()
    warm_ms = [a.elapsed_time(b) for a, b in warm]

    # HBM copy bandwidth measured on this device (1 GiB read + 1 GiB written per copy)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copies = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        copies.append((a, b))
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) / (statistics.median(a.elapsed_time(b) for a, b in copies) * 1e-3) / 1e9
    del src, dst
    props = torch.cuda.get_device_properties(0)
    cus = int(getattr(props, "multi_processor_count", 0))
    sclk_mhz = device_max_sclk_mhz()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    f_dense, f_reuse = dense_flops(w), reuse_flops(w)
    r_mean = statistics.fmean(reuse_ms)
    d_mean, d_med, d_min = statistics.fmean(dense_ms), statistics.median(dense_ms), min(dense_ms)
    exec_tflops = f_reuse / (r_mean * 1e-3) / 1e12       # the reuse step's executed rate: the value
    dense_eq = f_dense / (r_mean * 1e-3) / 1e12          # the dense work it stands in for, per second
    dense_tflops = f_dense / (d_mean * 1e-3) / 1e12
    rbytes = reuse_bytes_per_launch(w)
    # the instantiations the timed calls launch (bf16: float32 residual; d, G of the workload)
    sparse_name = f"sparse_ring_kernel<{w.d}, {w.group_size}, true>"
    dense_name = f"dense_bf16_kernel<{w.d}, 8>"
    traffic = load_traffic(sparse_name, w.name)
    mhz = load_clock(dense_name, w.name)
    peak_clk = cus * mhz * 1e6 * 4096 / 1e12 if cus and mhz else None
    out = {
        "metric": METRIC,
        "value": round(exec_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {workload_kind(w)}, B={w.B}, H={w.H}, d={w.d}, "
                               f"{w.dtype}, PDDP groups of {w.group_size}, keep {w.keep_permille / 10:g}% "
                               f"(k={w.k}), anchor every {A} steps, drift {w.drift} N(0,1) per step, "
                               f"residual R in float32",
                   "B": w.B, "H": w.H, "N": w.Nkv, "Nq": w.Nq, "d": w.d, "group_size": w.group_size, "k": w.k,
                   "anchor_every": A, "residual": "float32"},
        "step": f"one anchor period: mcs_group + mcs_anchor on step 0, mcs_sparse_attn on steps 1..{A - 1}",
        "value_is": "executed TFLOP/s of the reuse step (mcs_sparse_attn): 4*Nq*k*d*H FLOPs per call over the "
                    "mean cold call time",
        "reuse_ms_per_call": round(r_mean, 4),
        "reuse_ms_median": round(statistics.median(reuse_ms), 4),
        "reuse_ms_min": round(min(reuse_ms), 4),
        "reuse_executed_tflops": round(exec_tflops, 2),
        "reuse_executed_frac_bf16_peak": round(exec_tflops / PEAK_BF16_TFLOPS, 4),
        "reuse_dense_equivalent_tflops": round(dense_eq, 2),
        "reuse_bf16_residual_ms_per_call": round(statistics.fmean(r16_ms), 4) if r16_ms else None,
        "reuse_bf16_residual_ms_median": round(statistics.median(r16_ms), 4) if r16_ms else None,
        "dense_ms_per_call": round(d_mean, 4),
        "dense_ms_median": round(d_med, 4),
        "dense_ms_min": round(d_min, 4),
        "dense_tflops": round(dense_tflops, 2),
        "dense_frac_bf16_peak": round(dense_tflops / PEAK_BF16_TFLOPS, 4),
        "dense_frac_bf16_peak_median": round(f_dense / (d_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dense_frac_bf16_peak_min_time": round(f_dense / (d_min * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "speedup_reuse_vs_dense": round(d_mean / r_mean, 2),
        "cache": "flushed (512 MB overwrite before every timed call)" if not args.no_flush else "not flushed",
        "fidelity_rel_err_with_R": fid_r or None,
        "fidelity_rel_err_without_R": fid_nor or None,
        "fidelity_rel_err_stale_anchor_output": fid_stale or None,
        "fidelity_rel_err_block_sparse_recomputed": fid_bsa or None,
        "fidelity_rel_err_exact_selection_recomputed_without_R": fid_now or None,
        "block_sparse_ms_per_call": round(statistics.fmean(bsa_ms), 4),
        "block_select_ms_per_call": round(statistics.fmean(bsel_ms), 4),
        "drift_check_ms_per_call": round(statistics.fmean(drift_ms), 4),
        "drift_sampled_max_over_heads": fid_drift or None,
        "reuse_ms_warm_median": round(statistics.median(warm_ms), 4) if warm else None,
        "hbm_copy_gbs_measured": round(copy_gbs, 1),
        "device_cus": cus,
        "device_max_sclk_mhz": sclk_mhz,
        "peak_bf16_tflops_from_device": round(cus * sclk_mhz * 1e6 * 4096 / 1e12, 1) if cus and sclk_mhz else None,
        # the engine clock measured during timed dense launches (GRBM_GUI_ACTIVE per ns of a counter run
        # on the current kernel, profiles/clock.json) and the bf16 peak at that clock
        "sclk_mhz_measured_dense": mhz,
        "peak_bf16_tflops_at_measured_clock": round(peak_clk, 1) if peak_clk else None,
        "dense_frac_at_measured_clock": round(dense_tflops / peak_clk, 4) if peak_clk else None,
        "group_ms": round(statistics.fmean(group_ms), 4),
        "anchor_ms": round(statistics.fmean(anchor_ms), 4),
        "anchor_ms_single_pass": round(statistics.fmean(sp_ms), 4) if sp_ms else None,
        "period_effective_tflops_dense_equiv": round(A * f_dense / (wall / args.steps) / 1e12, 2),
        # the reuse kernel against the bf16 MFMA peak on the FLOPs it executes; its HBM rate is from
        # counter-measured bytes (traffic), and the rate of its logical gathers (most served by L2 and
        # the Infinity Cache, so above any HBM figure) is reported apart, never as a fraction
        "roofline": {"kernel": f"{sparse_name} (mcs_sparse_attn, reuse step)", "bound": "mfma",
                     "achieved": round(exec_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(exec_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "executed_flops_per_launch": f_reuse,
                     "frac_at_measured_clock": round(exec_tflops / peak_clk, 4) if peak_clk else None,
                     "traffic_gbs": round(traffic / (r_mean * 1e-3) / 1e9, 1) if traffic else None,
                     "traffic_frac": round(traffic / (r_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if traffic else None,
                     "logical_gather_bytes_per_launch": rbytes,
                     "logical_gather_gbs": round(rbytes / (r_mean * 1e-3) / 1e9, 1)},
        "roofline_dense": {"kernel": f"{dense_name} (mcs_dense_attn)", "bound": "mfma",
                           "achieved": round(dense_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(dense_tflops / PEAK_BF16_TFLOPS, 4),
                           "traffic": load_traffic(dense_name, w.name)},
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, host[0], host[1], args.cpu_heads)
        cb["gpu_over_oracle_reuse"] = round(cb["reuse_ms_per_call_extrapolated"] / r_mean, 1)
        cb["gpu_over_oracle_dense"] = round(cb["dense_ms_per_call_extrapolated"] / d_mean, 1)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
