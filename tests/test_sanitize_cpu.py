"""Sanitizer runs on the host (no GPU): the C oracle and the library's C-ABI
validation built with AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/fp8q_oracle.c) with a driver that runs every function on
  small ragged inputs and checks a few facts any correct build satisfies.
* The host code of the C-ABI layer (fp8_precision_quant_amd/csrc/api.hip,
  compiled for the host only) linked with launcher stand-ins that abort if
  reached, and a driver that calls every entry point with arguments its
  validation must reject, checking each status.  No call reaches a device.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd, **kw):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "fp8q_oracle.c"), "-o", exe, "-lm"],
         cwd=str(tmp_path))
    r = _run([exe], cwd=str(tmp_path), env=ENV, timeout=300)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-g", "-std=c++17", "-Wno-unused-command-line-argument"]
    objs = []
    for src in (os.path.join(ROOT, "fp8_precision_quant_amd", "csrc", "api.hip"),
                os.path.join(SAN, "launcher_stubs.cpp"), os.path.join(SAN, "api_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--cuda-host-only", *flags, *san, "-c", src, "-o", obj], cwd=str(tmp_path))
        objs.append(obj)
    exe = str(tmp_path / "api_driver")
    _run([HIPCC, *san, *objs, "-o", exe], cwd=str(tmp_path))
    r = _run([exe], cwd=str(tmp_path), env=ENV, timeout=120)
    assert "all validation cases passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
