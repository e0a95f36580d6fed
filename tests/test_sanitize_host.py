"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds tests/sanitize/abi_checks.cpp against the library sources with both sanitizers on
the host half (the device half is compiled unoptimised and never launched) and runs it:
codebook, polar-grid and codec-table builds into exactly sized buffers, cache sizes at
the shape limits, and every device entry point's host-side validation.  A sanitizer
report or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vector_quantization_rope_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    objs = []
    for src, extra in (("tq_host.cpp", []),
                       ("tq_device.hip", ["-x", "hip", "--offload-arch=gfx950", "-Xarch_device", "-O0"]),
                       (os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), [])):
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, log = _run([HIPCC, *extra, "-O1", "-g", "-std=c++17", *SAN, "-c", path, "-o", obj])
        assert rc == 0, log[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_checks")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe])
    assert rc == 0, log[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, log = _run([exe], env=env, timeout=600)
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
    assert rc == 0, log[-4000:]
    assert "0 failed" in log, log[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
