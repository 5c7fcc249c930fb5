"""Sanitizer leg of the CPU tests: the fp64 oracle and the library's host code (argument
checks, the cu_seqlens and block-layout validators, launch setup) rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer, and the CPU tests that exercise them run
against those builds in a child process.  Any sanitizer report aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(cmd):
    path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"sanitizer runtime not found ({' '.join(cmd)})")
    return path


def _child(env, tests):
    env = dict(os.environ, **env, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return tail


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    import oracle
    so = oracle.build(force=True, sanitize=True, path=str(tmp_path / "liboracle_asan.so"))
    tail = _child({"PFA_ORACLE_LIB": so, "LD_PRELOAD": _runtime(["gcc", "-print-file-name=libasan.so"])},
                  ["tests/test_oracle_pins.py", "tests/test_workloads.py", "tests/test_tolerance.py"])
    print(tail.strip().splitlines()[-1])


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    from packed_varlen_flash_amd import build
    so = build.build(sanitize_host=True, path=str(tmp_path / "libpfa_asan.so"))
    rt = _runtime(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    tail = _child({"PFA_LIB": so, "LD_PRELOAD": rt}, ["tests/test_abi_cpu.py"])
    print(tail.strip().splitlines()[-1])
