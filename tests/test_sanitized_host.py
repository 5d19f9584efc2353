"""The oracle (oracle/svo.c) and the library's host code (descriptor and
argument validation, workspace sizing, the C ABI's entry points up to any
launch) built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer,
and the CPU tests of both run against those builds in a child process with
the sanitizer runtime preloaded.  The library's device code is compiled
without optimisation in that build (the CPU tests make no launch; it is
there so that the library loads).  A report from either sanitizer ends the
child with an error, which fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CSRC = os.path.join(ROOT, "lossless_draft_verification_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("specverify.hip", "planner.hip", "compact.hip", "stream_read.hip")]
# the oracle's CPU tests that run in seconds (the statistical ones are left to the plain run)
ORACLE_TESTS = ["tests/test_oracle_rules.py", "tests/test_oracle_filter.py", "tests/test_oracle_stats.py",
                "tests/test_oracle_block.py", "tests/test_oracle_plan.py", "tests/test_oracle_compact.py",
                "tests/test_oracle_philox.py"]


def _runtime():
    if not os.path.exists(CLANG):
        pytest.skip("no clang")
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = rt.stdout.strip()
    if rt.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no AddressSanitizer runtime")
    return path


def test_host_code_and_oracle_under_sanitizers(tmp_path):
    rt = _runtime()
    oracle_lib = str(tmp_path / "libsvo_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", oracle_lib,
                    os.path.join(ROOT, "oracle", "svo.c"), "-lm"], check=True)
    lib = str(tmp_path / "libspecverify_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_device", "-O0", *san,
                    "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", lib], check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=rt, SV_TEST_LIB=lib, SV_TEST_ORACLE_LIB=oracle_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_host.py", *ORACLE_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
