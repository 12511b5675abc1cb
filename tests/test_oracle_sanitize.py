"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_check.c calls every oracle entry point on buffers sized
exactly as each contract states, with the degenerate cases (empty contexts,
k above the visible count, invalid slots, unallocated pages); this test
builds it together with oracle.c for the host with both sanitizers and
requires a clean run.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           os.path.join(ORACLE, "oracle.c"), os.path.join(ORACLE, "sanitize_check.c"),
           "-I", ORACLE, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr
    # the environment is passed on unchanged apart from the sanitizer options
    # (a preloaded library ahead of the ASan runtime is tolerated)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
