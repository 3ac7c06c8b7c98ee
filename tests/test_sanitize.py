"""Host-code sanitizer run (CPU only): the C ABI's argument validation, dispatch and per-device
state (api.cpp, launch_attr.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer (host
pass only, linked with the ordinary kernel objects), exercised by the ABI tests in a subprocess
that preloads clang's ASan runtime and loads that build through RBA_LIBRARY.  Any report aborts
the subprocess (halt_on_error), so the test fails on the first one."""

import os
import subprocess
import sys

import pytest

from transformer_attention_learned_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_checks_under_asan_and_ubsan():
    try:
        lib = build.build_sanitized()
        rt = build.sanitizer_runtime()
    except RuntimeError as e:  # no ROCm toolchain here
        pytest.skip(f"sanitizer build unavailable: {e}")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "host code not instrumented"
    env = dict(os.environ, RBA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # every ABI test but the one that checks the error for a missing library
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-k", "not binding_refuses"],
                       env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-4000:] + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail
