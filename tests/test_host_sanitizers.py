"""The library's host code under the compiler's sanitizers (CPU only).

The size-class cache (csrc/cache.cpp) and the expert store and miss pipeline
with its I/O threads and event rings (csrc/pipeline.cpp) are built unchanged
with g++ against a host-only stand-in for the HIP runtime
(tests/sanitize/stub, tests/sanitize/hip_stub.cpp: streams are worker threads
that run their queues in order, copies are asynchronous, events follow HIP's
record / query / wait semantics), and driven by tests/sanitize/host_driver.cpp:
random cache sequences checked against the cache's invariants, store reads,
and pipeline layer steps whose routed rows are checked on the compute stream
after the waits that moe_pipeline_prepare enqueues.

Two builds: address + undefined-behaviour sanitizers, and the thread
sanitizer (a copy that lands in a slot while a forward still reads it, or a
forward that reads a slot before its install completed, is a data race between
stream threads).  Either build must finish with no sanitizer report and every
driver check passing.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "sanitize")
CSRC = os.path.join(os.path.dirname(HERE), "quantized_routed_expert_softmax_amd", "csrc")
SOURCES = [os.path.join(CSRC, "cache.cpp"), os.path.join(CSRC, "pipeline.cpp"),
           os.path.join(SAN, "hip_stub.cpp"), os.path.join(SAN, "host_driver.cpp")]

RUNS = 10

BUILDS = {
    "address_undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
    "thread": ["-fsanitize=thread"],
}


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("kind", sorted(BUILDS))
def test_host_code_under_sanitizer(kind, tmp_path):
    exe = str(tmp_path / f"host_driver_{kind}")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *BUILDS[kind],
           "-I", os.path.join(SAN, "stub"), "-I", SAN, *SOURCES, "-pthread", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=66"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=66"
    env["TSAN_OPTIONS"] = "halt_on_error=0:exitcode=66"
    # several runs: stream threads interleave differently each time (a fill that
    # completed between the cache's check and the pipeline's own once turned a
    # full class into a spurious MOE_E_NO_SLOT in about one run in fifty)
    for _ in range(RUNS):
        run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env, cwd=str(tmp_path))
        out = run.stdout + run.stderr
        assert run.returncode == 0, out[-6000:]
        assert "host driver: ok" in run.stdout
        for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                       "ERROR: LeakSanitizer"):
            assert marker not in out, out[-6000:]
