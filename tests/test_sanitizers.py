"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize are built with -fsanitize=address,undefined and run:
plan_driver.cpp sweeps the library's host-side shape validation, planning and call checks
(kda_plan.cpp, the code every entry point runs before launching) over valid, invalid and
limit-sized shapes; oracle_driver.c runs the fp64 oracle over small inputs of every layout and
option.  Any sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]


def build_and_run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if "asan" in res.stderr.lower() and "cannot find" in res.stderr.lower():
            pytest.skip("sanitizer runtime not installed")
        raise AssertionError(f"build failed:\n{' '.join(cmd)}\n{res.stderr}")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, f"{exe} failed ({run.returncode}):\n{run.stdout[-3000:]}\n{run.stderr[-3000:]}"
    assert "runtime error" not in run.stderr, run.stderr[-3000:]
    return run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_plan_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_san")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-I/opt/rocm/include",
           f"-I{ROOT}/kimi_delta_attention_chunk_amd/csrc",
           f"{ROOT}/tests/sanitize/plan_driver.cpp",
           f"{ROOT}/kimi_delta_attention_chunk_amd/csrc/kda_plan.cpp", "-o", exe]
    out = build_and_run(cmd, exe)
    assert "failures 0" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c11", *SAN, f"{ROOT}/tests/sanitize/oracle_driver.c",
           f"{ROOT}/oracle/kda_oracle.c", "-o", exe, "-lm"]
    out = build_and_run(cmd, exe)
    assert "failures 0" in out
