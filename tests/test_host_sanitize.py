"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The CPU oracle (oracle/oracle.c) and the plan code (tp_plan.cpp) are compiled
with -fsanitize=address,undefined by gcc/g++ (host compilers only: no device
code is built here) together with tests/host_sanitize_main.cpp, which drives
them over small and benchmark-sized shapes, valid and invalid. The plan code
asks the built library for its two kernel geometries (host functions in the
HIP sources), so the program links against libtpdecode.so for those; the
interface functions themselves come from the sanitized object. The run must
exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "row_gemv_reduction_amd")
LIB = os.path.join(PKG, "libtpdecode.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no host compiler")
def test_oracle_and_plan_under_asan_ubsan(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libtpdecode.so is not built; run __graft_entry__.build() first")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc")]
    oracle_o = str(tmp_path / "oracle.o")
    plan_o = str(tmp_path / "tp_plan.o")
    main_o = str(tmp_path / "main.o")
    exe = str(tmp_path / "host_sanitize")
    _run(["gcc", "-std=c99", *SAN, "-c", os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_o])
    _run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(PKG, "csrc", "tp_plan.cpp"), "-o", plan_o])
    _run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(ROOT, "tests", "host_sanitize_main.cpp"),
          "-o", main_o])
    _run(["g++", *SAN, main_o, plan_o, oracle_o, "-o", exe, "-L" + PKG, "-ltpdecode",
          "-Wl,-rpath," + PKG, "-lpthread", "-lm"])
    env = dict(os.environ)
    # the HIP runtime the library links keeps allocations until exit by design
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = _run([exe], env=env)
    assert "host sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
