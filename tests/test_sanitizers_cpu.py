"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host code in api.hip (argument validation, workspace sizing,
  launch geometry, the static-scratch lookup) is rebuilt with both sanitizers
  on its host pass only (the device code is not instrumented) and linked with
  the regular objects of the other sources; the whole CPU ABI suite
  (test_library_cpu.py) then runs against it.
* The oracle is rebuilt by gcc with both sanitizers and runs its pins
  (test_oracle_pins.py, test_oracle_backward_pins.py).

Each suite runs in a child process with the matching sanitizer runtime
preloaded (the interpreter itself is not instrumented); a sanitizer report
halts the child and fails the test.  A probe in the same environment checks
that the sanitized builds, not the regular ones, are the ones loaded.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(args, env):
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def _mapped(env, load, name):
    probe = (f"import os, sys; sys.path.insert(0, {ROOT!r}); {load}; "
             f"print(any({name!r} in line for line in open('/proc/self/maps')))")
    return _child(["-c", probe], env).strip().splitlines()[-1] == "True"


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from compressed_attention_kv_amd import build as hipbuild
    try:
        so = hipbuild.build_sanitized(str(tmp_path))
        rt = hipbuild.asan_runtime()
    except FileNotFoundError as e:  # the regular build has not run in this tree
        pytest.skip(str(e))
    env = dict(os.environ, **OPTS, LD_PRELOAD=rt, CAKV_TEST_LIBRARY=so)
    assert _mapped(env, "import compressed_attention_kv_amd as c; c.load_library(os.environ['CAKV_TEST_LIBRARY'])",
                   "libcakv_sanitized.so")
    out = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_library_cpu.py"], env)
    assert " passed" in out and " failed" not in out


def test_oracle_under_asan_and_ubsan(tmp_path):
    import oracle
    so = oracle.build_sanitized(str(tmp_path))
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isfile(rt), "gcc's libasan was not found"
    env = dict(os.environ, **OPTS, LD_PRELOAD=rt, CAKV_ORACLE_LIBRARY=so)
    assert _mapped(env, "import oracle; oracle._load()", "libcakv_oracle_sanitized.so")
    out = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
                  "tests/test_oracle_backward_pins.py"], env)
    assert " passed" in out and " failed" not in out
