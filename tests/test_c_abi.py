"""The C ABI from C (not gpu): tests/c_abi_check.c includes include/mcs.h
under gcc -std=c99 -pedantic -Werror, links the built libmcs.so and checks
the host-only calls (version, status strings, workspace sizes, host-side
argument checks, the empty-problem no-op)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_attention_video_pddp_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c_caller_compiles_links_and_runs(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libmcs.so")):
        pytest.fail("libmcs.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "c_abi_check")
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
                    "-L", LIBDIR, "-lmcs", "-Wl,-rpath," + LIBDIR, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
