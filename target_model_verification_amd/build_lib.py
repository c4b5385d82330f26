"""Builds libspecverify.so (HIP kernels for gfx950 + host runtime) in place.

Usage: python -m target_model_verification_amd.build_lib [--jobs N]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["pass.hip", "retile.hip", "misc.hip", "noalloc.hip", "plan_check.cpp", "spec_verify.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 VALU forms are disabled for all device code
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-Wno-unused-but-set-variable"]


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(jobs: int = 4) -> str:
    with tempfile.TemporaryDirectory() as td:
        objs = [os.path.join(td, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max(1, jobs)) as ex:
            list(ex.map(lambda a: _compile(*a), zip(SOURCES, objs)))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    jobs = 4
    if "--jobs" in sys.argv:
        jobs = int(sys.argv[sys.argv.index("--jobs") + 1])
    print(build(jobs))
