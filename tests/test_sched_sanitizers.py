"""The step planner (host C++, csrc/sched.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer (host compiler only; no GPU code is built)
and driven through its C ABI by tests/sanitize/sched_driver.cpp over many
random steps: admissions, prefix-cache hits, chunked prefill, preemption
when the pool runs dry, early finishes. Any out-of-bounds access, use after
free, leak or undefined behaviour fails the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_kv_amd", "csrc")


def test_planner_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "sched_driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "sched.cpp"), os.path.join(ROOT, "tests", "sanitize", "sched_driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in (r.stderr or ""):
        pytest.skip("the host compiler has no sanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "planner driver ok" in run.stdout
