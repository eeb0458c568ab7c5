"""The host-side ABI checks (tests/test_abi_cpu.py) rerun against a build of the C ABI
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
(configuration validation, arena planning, tensor table, argument checks), in a child
Python process that preloads the sanitizer runtime.  Any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    from gpt_pretraining_step_train_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), GPTMI_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=550)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
