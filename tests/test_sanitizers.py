"""CPU sanitizer tier: the fp64 oracle and the launch planner built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code only) and
run over small random and edge-case arguments by tests/sanitize/driver.cpp.
Any sanitizer report, or a failed identity in the driver, fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_oracle_and_planner_under_asan_ubsan(tmp_path):
    ref_o = str(tmp_path / "linattn_ref.o")
    plan_o = str(tmp_path / "linattn_plan.o")
    drv_o = str(tmp_path / "driver.o")
    exe = str(tmp_path / "sanitized")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "sequence_mixing_amd", "csrc"),
           "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    cmds = [
        ["gcc", "-std=c99", *SAN, "-ffp-contract=off", "-c", os.path.join(ROOT, "oracle", "linattn_ref.c"),
         "-o", ref_o],
        ["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(ROOT, "sequence_mixing_amd", "csrc", "linattn_plan.cpp"),
         "-o", plan_o],
        ["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), "-o", drv_o],
        ["g++", *SAN, drv_o, plan_o, ref_o, "-o", exe, "-lm", "-lpthread"],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(c)}\n{r.stderr}"
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms, "the binary is not instrumented"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "ok" in r.stdout
