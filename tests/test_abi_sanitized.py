"""The host-only ABI tests again, against a build of the library whose host
code runs under AddressSanitizer and UndefinedBehaviorSanitizer (device code
unchanged), so that an out-of-bounds access, use after free or undefined
behaviour in the validation, workspace-layout or launch-cache code fails
the run instead of passing silently. No GPU is needed: every call in those
tests returns before any device work."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_qgemv_build", os.path.join(ROOT, "block_quant_gemv_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(900)
def test_abi_host_tests_under_asan_and_ubsan():
    b = _build_module()
    try:
        lib = b.build_sanitized()
    except RuntimeError as e:  # no ROCm toolchain here
        pytest.skip(f"cannot build the sanitized library: {e}")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    rt = b.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env.update(QGEMV_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_abi_lib.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
