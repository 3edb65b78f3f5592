"""Sanitizer builds on the CPU (no GPU is touched).

* The oracle's C code (oracle/m2_oracle.c) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer and loaded in place of the regular build (M2_ORACLE_LIB) by a
  subprocess that runs the oracle pin tests with the ASan runtime preloaded.
* The host side of the C ABI (m2_api.cpp: argument checks, handle bookkeeping, the stack
  table, the panel and no-alloc entry points) built with clang's AddressSanitizer and UBSan
  for host code only (hipcc -Xarch_host), linked with the regular device objects into a
  driver (tests/sanitize/host_checks.cpp) that calls every entry point with bad arguments
  and checks the statuses; every call is rejected before any HIP call.
* A canary: a planted heap overflow in a throwaway program must be reported, so a silent
  harness cannot pass the two tests above."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's libasan.so not found")
    return path


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    exe = str(tmp_path / "canary")
    subprocess.check_call(["gcc", "-O0", "-g", "-fsanitize=address", os.path.join(ROOT, "tests/sanitize/canary.c"),
                           "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env={**os.environ, **SAN_ENV})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle/m2_oracle.c"), "-o", so, "-lm"])
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": _gcc_asan_runtime(), "M2_ORACLE_LIB": so, "OMP_NUM_THREADS": "4"}
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests/test_oracle_pins.py"), "-x", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out


def test_host_checks_under_asan(tmp_path):
    objs = [os.path.join(ROOT, "full_duplex_speech_mamba2_amd/_build/%s.o" % n)
            for n in ("decode", "fused", "prefill", "attention")]
    if not os.path.exists(HIPCC) or not all(os.path.exists(o) for o in objs):
        pytest.skip("hipcc or the device objects of the regular build are missing (run __graft_entry__.build())")
    csrc = os.path.join(ROOT, "full_duplex_speech_mamba2_amd/csrc")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "m2_api.o")
    drv = str(tmp_path / "host_checks.o")
    exe = str(tmp_path / "host_checks")
    subprocess.check_call([HIPCC, "-x", "hip", "-c", os.path.join(csrc, "m2_api.cpp"), "-o", api,
                           "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
                           "-I" + os.path.join(ROOT, "include"), "-I" + csrc] + san)
    subprocess.check_call([HIPCC, "-c", os.path.join(ROOT, "tests/sanitize/host_checks.cpp"), "-o", drv,
                           "-std=c++17", "-O1", "-g", "-I" + os.path.join(ROOT, "include")] + san)
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-o", exe, drv, api] + objs + san)
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1", "UBSAN_OPTIONS": SAN_ENV["UBSAN_OPTIONS"]}
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "0 failed" in r.stdout and "Sanitizer" not in out, out[-3000:]
