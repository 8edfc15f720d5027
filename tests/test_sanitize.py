"""The library's host code under AddressSanitizer and UBSan, on the CPU.

Builds the sanitizer build of libtpla (tensor_latent_decode_amd/
build_sanitize.py: argument checks, split planning, the split cost model and
the rest of the host side instrumented) and runs the C-ABI tests, with the
split-suggestion fuzz, against it in a child interpreter that preloads the
sanitizer runtime.  Any sanitizer report ends that child with a failure.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_address_and_ub_sanitizers():
    sys.path.insert(0, ROOT)
    from tensor_latent_decode_amd import build_sanitize

    lib = build_sanitize.build()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build_sanitize.runtime_path(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "TPLA_LIB": lib,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
