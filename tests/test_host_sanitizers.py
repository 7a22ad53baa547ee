"""The library's host code (argument validation, status and error text, workspace
sizing, stream and timer bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer.

A second build of the same sources instruments the host pass only, and the C-ABI tests of
test_abi.py run against it in a child process with the ASan runtime preloaded; any report
from either sanitizer ends that process with a non-zero status. CPU only: no call reaches
a kernel."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "h2o_sparse_attention_amd"))
import build as h2o_build  # noqa: E402


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    try:
        runtime = h2o_build.asan_runtime()
    except (RuntimeError, OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no ASan runtime: {e}")
    lib = h2o_build.build_host_sanitized(str(tmp_path_factory.mktemp("san")))
    return lib, runtime


def test_sanitized_build_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE,
                          text=True, check=True).stdout
    assert "__asan_report_load" in syms
    assert "__ubsan_handle_" in syms


def test_abi_suite_clean_under_asan_and_ubsan(sanitized_lib):
    lib, runtime = sanitized_lib
    env = dict(os.environ)
    env.update(
        H2O_LIB_PATH=lib,
        LD_PRELOAD=runtime,
        # leaks: the interpreter and the HIP runtime keep allocations until exit by design;
        # the mismatch and ODR checks trip on uninstrumented libraries in the process
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86:"
                     "alloc_dealloc_mismatch=0:detect_odr_violation=0",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87",
    )
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    out = p.stdout
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
