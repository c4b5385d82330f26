"""The library's host runtime (configuration and plan checks, tree-expansion
and lookahead policies, null-handle calls) built with AddressSanitizer on the
host side only and driven by tests/host_asan/driver.cpp; the device entry
points are stubs (tests/host_asan/stubs.cpp), so nothing runs on a GPU.
Skipped when hipcc is not installed."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "target_model_verification_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
         "-I" + os.path.join(ROOT, "include")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_runtime_under_address_sanitizer():
    with tempfile.TemporaryDirectory() as td:
        srcs = [os.path.join(CSRC, "spec_verify.cpp"), os.path.join(CSRC, "plan_check.cpp"),
                os.path.join(ROOT, "tests", "host_asan", "stubs.cpp"),
                os.path.join(ROOT, "tests", "host_asan", "driver.cpp")]
        objs = []
        procs = []
        for s in srcs:
            o = os.path.join(td, os.path.basename(s) + ".o")
            objs.append(o)
            procs.append(subprocess.Popen([HIPCC] + FLAGS + ["-c", s, "-o", o], stdout=subprocess.PIPE,
                                          stderr=subprocess.STDOUT, text=True))
        for p in procs:
            out, _ = p.communicate()
            assert p.returncode == 0, out[-3000:]
        exe = os.path.join(td, "host_check")
        r = subprocess.run([HIPCC, "-Xarch_host", "-fsanitize=address", "-o", exe] + objs, capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
        assert r.returncode == 0, r.stderr[-4000:]
        assert "0 failure(s)" in r.stderr
