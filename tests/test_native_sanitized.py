"""CPU: the host runtime (validation, planning, staging ring) and the C oracle, built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

* tests/native/host_runtime_check.cpp links kamera_api.cpp and kamera_host.cpp against a
  counting stand-in for the HIP runtime: the staging ring is allocated once per device, no
  compute call allocates, frees or waits on the host after that, a full ring answers
  KAMERA_ERR_BUSY with nothing enqueued, capture is refused, rejected calls enqueue nothing.
* tests/native/oracle_check.c drives every code path of oracle/kamera_oracle.c.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "position_invariant_kv_kamera_amd" / "csrc"
NATIVE = ROOT / "tests" / "native"
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_runtime_under_sanitizers(tmp_path):
    exe = tmp_path / "host_runtime_check"
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          str(NATIVE / "host_runtime_check.cpp"), str(CSRC / "kamera_api.cpp"),
          str(CSRC / "kamera_host.cpp"), "-o", str(exe)])
    res = _run([str(exe)], env=ENV, timeout=300)
    print(res.stdout)
    assert "0 failure(s)" in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", str(ROOT / "oracle" / "kamera_oracle.c"),
          str(NATIVE / "oracle_check.c"), "-lm", "-o", str(exe)])
    res = _run([str(exe)], env=ENV, timeout=300)
    print(res.stdout)
    assert "0 failure(s)" in res.stdout
