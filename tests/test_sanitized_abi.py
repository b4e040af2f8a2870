"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer: the host code of the library (api.cpp: validation,
overflow checks, workspace layout, dispatch up to the first HIP call) built
with both sanitizers, and tests/test_abi.py run against it in a child Python
process with the sanitizer runtime preloaded. Every refusal path runs; a
sanitizer report fails the child (halt_on_error) and this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    if not shutil.which("g++"):
        return None
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_checks_clean_under_asan_ubsan(tmp_path):
    from int4_quantized_gemm_amd import build_lib
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    try:
        lib = build_lib.build_sanitized_api(str(tmp_path))
    except FileNotFoundError as e:
        pytest.skip(str(e))
    code = (
        "import sys; sys.path.insert(0, {root!r})\n"
        "import int4_quantized_gemm_amd._lib as L\n"
        "L.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main([{tests!r}, '-q', '-x', '-p', 'no:cacheprovider']))\n"
    ).format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
