"""The C ABI's host code (argument validation, the workspace carving of every
layout, the timing hook, return-code texts) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU: tests/sanitize/host_checks.cpp
drives every entry point down its rejection paths and sizes every workspace
over a grid of arguments, before any HIP call is made.  The sanitizers
instrument host code only (each -fsanitize= follows -Xarch_host); the device
code is compiled as usual and never runs here.  The executable is cached
under tests/sanitize/_build keyed by the sources' digest, so only the first
run after a source change pays for the build (about two minutes)."""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "inverse_root_preconditioning_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")
OUTDIR = os.path.join(ROOT, "tests", "sanitize", "_build")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _digest():
    h = hashlib.sha256(" ".join(FLAGS).encode())
    paths = [DRIVER, os.path.join(ROOT, "include", "shampoo.h")]
    paths += sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".h", ".hip")))
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_address_and_undefined_behavior_sanitizers():
    exe = os.path.join(OUTDIR, f"host_checks_{_digest()}")
    if not os.path.exists(exe):
        if os.path.isdir(OUTDIR):
            shutil.rmtree(OUTDIR)
        os.makedirs(OUTDIR)
        cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), DRIVER,
                                 os.path.join(CSRC, "shampoo.hip"), "-o", exe + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=1200)
        assert res.returncode == 0, res.stderr[-4000:]
        os.replace(exe + ".tmp", exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, (res.returncode, res.stdout[-2000:], res.stderr[-6000:])
    assert "host checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
