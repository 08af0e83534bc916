"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI's host side (argument validation, the batched plan builders, the
size queries, the error buffer) is built with -fsanitize=address,undefined
(host code only; the device code is unchanged) and the whole CPU ABI suite
(tests/test_abi_cpu.py) runs against that build in a child Python with the
ASan runtime preloaded.  Any sanitizer report ends the child with an error.
No GPU is touched: every call in that suite returns before the first HIP call.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers():
    from quantized_matmul_qgemv_amd import build as B
    try:
        lib = B.build_host_sanitized()
        rt = B.asan_runtime()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    env = dict(os.environ)
    env.update({
        "QMM_LIBRARY": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87",
        "HIP_VISIBLE_DEVICES": "",
    })
    probe = subprocess.run([sys.executable, "-c", "from quantized_matmul_qgemv_amd import _lib; "
                            "_lib.lib(); print(_lib.LIB_PATH)"], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out, out[-3000:]
