"""The library's host code (launch planning and every argument check) under
AddressSanitizer and UndefinedBehaviorSanitizer: api.hip is compiled with
the sanitizers on its host side only (-Xarch_host), linked with the fuzz
driver tests/sanitize/host_fuzz.cpp (also instrumented) and the kernels of
the built libkvq.so, and run on the CPU.  The driver only plans and only
makes calls that are refused before anything is enqueued, so nothing
launches; a sanitizer report aborts it (non-zero exit)."""
import os
import shutil
import subprocess
import sys

import pytest

from tests.helpers import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_kivi_amd")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(_hipcc()) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_planner_and_checks_under_asan_ubsan(tmp_path):
    ensure_built()
    sys.path.insert(0, ROOT)
    from decode_attention_kivi_amd import build as B
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "host_fuzz.o")
    exe = str(tmp_path / "host_fuzz")
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    subprocess.run([_hipcc(), *B.COMMON, "-g", "-O1", *host_san, "-c", os.path.join(B.CSRC, "api.hip"),
                    "-o", api_o], check=True, capture_output=True)
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "sanitize", "host_fuzz.cpp"), "-o", drv_o],
                   check=True, capture_output=True)
    # the instrumented api.o defines the entry points the driver calls; the
    # kernels and launchers come from libkvq.so
    subprocess.run([_hipcc(), f"--offload-arch={B.ARCH}", *host_san, drv_o, api_o, "-L", PKG, "-lkvq",
                    f"-Wl,-rpath,{PKG}", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host fuzz:" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
