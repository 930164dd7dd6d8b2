"""The oracle's pins and the C ABI's host validation under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

Two builds made for this: the C oracle compiled by gcc with
-fsanitize=address,undefined (oracle.build.build_sanitized), and the HIP
library whose host code (msd_api.cpp: validation, dispatch, workspace
bookkeeping) is compiled with the same sanitizers by hipcc, host side only
(weight_only_quantized_msd_amd.build.build_host_sanitized).  Each test file
then runs in a child process that preloads the matching sanitizer runtime
(gcc's libasan for the oracle, clang's for the library; one process cannot
hold both) and selects the sanitized build through MSD_ORACLE_LIB / WQBMM_LIB.
Any sanitizer report aborts the child (-fno-sanitize-recover=all), which
fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + args,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    return r.stdout


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_ubsan():
    rt = _gcc_asan()
    if rt is None:
        pytest.skip("gcc's libasan is not installed")
    from oracle.build import build_sanitized
    lib = build_sanitized()
    out = _run({"LD_PRELOAD": rt, "MSD_ORACLE_LIB": lib},
               ["tests/test_oracle_pins.py", "-k", "not outlier_m128 and not pages_sample_m1"])
    assert "failed" not in out


def test_boundary_validation_under_asan_ubsan():
    rts = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    from weight_only_quantized_msd_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    out = _run({"LD_PRELOAD": rts[0], "WQBMM_LIB": lib}, ["tests/test_boundary.py"])
    assert "failed" not in out
