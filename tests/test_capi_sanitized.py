"""The C-ABI's host validation layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The build step makes a second copy of the library whose host code (lsa_api.hip: argument checks,
offset scans, error messages) is compiled with both sanitizers; the GPU code is the same. The
host-side C-ABI tests (test_capi_host.py) then run against that copy in a subprocess with the
sanitizer runtime preloaded: every rejected call must behave as in the product build, with no
sanitizer report. No GPU is needed; nothing reaches the device.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        out = subprocess.run(["/opt/rocm/llvm/bin/clang++", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def test_host_validation_under_sanitizers():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or clang sanitizer runtime in this environment")
    sys.path.insert(0, ROOT)
    from sparse_kv_retrieval_amd import build as B
    pkg_parent = os.path.dirname(B.build_sanitized_host())
    # run from the sanitized copy's directory, so that it (not the product package) is found first
    env = dict(os.environ, PYTHONPATH=pkg_parent, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the subprocess must load the sanitized copy, not the product library
    probe = subprocess.run([sys.executable, "-c", "from sparse_kv_retrieval_amd import lsa; print(lsa.LIB_PATH)"],
                           cwd=pkg_parent, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().startswith(pkg_parent), probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "--import-mode=append", "--rootdir", ROOT, os.path.join(ROOT, "tests", "test_capi_host.py")],
                       cwd=pkg_parent, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report + "\nRC=" + str(r.returncode)
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report
