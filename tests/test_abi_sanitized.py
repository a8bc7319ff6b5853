"""The C-ABI host validation under AddressSanitizer and UndefinedBehaviorSanitizer.

pisa_api.hip is rebuilt with both sanitizers on its host code, linked with the
normal objects of the other sources, and the whole host-side ABI suite
(tests/test_abi.py: exported symbols, struct layout, every acceptance and
rejection path of the argument checks -- none of which launches a kernel) runs
against it in a child process with the sanitizer runtime preloaded. Any report
(heap or stack overflow, use after free, signed overflow, misaligned access,
invalid shift, ...) aborts the child and fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_passes_under_host_sanitizers():
    from block_sparse_long_pisa_amd import build

    try:
        lib = build.build_sanitized()
        runtime = build.sanitizer_runtime()
    except RuntimeError as e:  # no ROCm toolchain on this machine
        pytest.skip(str(e))
    env = dict(os.environ)
    env["PISA_LIBRARY"] = lib
    env["LD_PRELOAD"] = " ".join(x for x in (runtime, env.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
