"""The host side of libcva under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Builds the library with its host C++ instrumented (validation, metadata, tile
schedules, block placement, C ABI; the HIP kernels are not instrumented), then
runs the host test files against it in a child process with the sanitizer
runtimes preloaded and the planner on 8 threads (the threaded row and block
passes run for 32768 or more local rows: the sparse-mask batch).  Any
sanitizer report aborts the child (no recovery), so the run must end clean.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_capi_host.py", "tests/test_placement_host.py", "tests/test_plan_tables.py"]


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], stdout=subprocess.PIPE,
                           text=True, timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None or shutil.which("g++") is None:
        pytest.skip("gcc sanitizer runtimes not available")
    from context_varlen_attention_amd.build import build_host_sanitized
    lib = build_host_sanitized(str(tmp_path / "libcva_sanitized.so"))
    env = dict(os.environ, CVA_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}", CVA_PLAN_THREADS="8",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *HOST_TESTS], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
