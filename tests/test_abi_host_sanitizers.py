"""The host side of the C ABI (argument validation, descriptors, workspace
layouts, launch set-up) under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is built with both on its host code (``python -m
paged_kv_gqa_cache_amd.build --host-sanitizers``) and tests/test_abi.py runs
against it in a child process with the ASan runtime preloaded.  No GPU: every
call in test_abi.py returns from validation before touching a device."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime() -> str | None:
    if not os.path.exists(CLANG):
        return None
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isfile(path) else None


def _sanitized_lib() -> str:
    from paged_kv_gqa_cache_amd import build
    lib = build.HOSTSAN_LIB
    newest = max(os.path.getmtime(p) for p in build.sources() + [build.__file__])
    if not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        build.build(verbose=False, host_sanitizers=True)
    return lib


@pytest.mark.timeout(600)
def test_abi_validation_is_clean_under_host_sanitizers():
    runtime = _asan_runtime()
    if runtime is None or not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    lib = _sanitized_lib()
    # the host code carries the sanitizers' checks
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, LD_PRELOAD=runtime, PAGEDKV_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the sanitized library, with the ASan runtime live
    probe = subprocess.run(
        [sys.executable, "-c",
         "import ctypes; ctypes.CDLL(None).__asan_address_is_poisoned; "
         "from paged_kv_gqa_cache_amd import abi; print(abi.lib()._name)"],
        cwd=ROOT, env=env, capture_output=True, text=True)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().endswith("libpagedkv_hostsan.so")
    run = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True)
    log = run.stdout + run.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert run.returncode == 0, log[-4000:]
    assert " passed" in log
