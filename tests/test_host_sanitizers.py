"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the C ABI shim's argument checks and
the host block manager (its FIFO ring, reference counts and sequence map;
"How does paged attention work (in detail)", sections 3.2 and 4.1).

* bm_sanitize: seeded random traces of every pa_bm_* call with the
  manager's invariants checked after each step, leak checking on;
* the ABI and block-manager tests of this directory, run again in a child
  Python process that loads the instrumented build (PA_LIB) with the ASan
  runtime preloaded.  Any sanitizer report fails the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    from paged_kv_cache_78_amd import build, build_sanitized
    if not os.path.exists(os.path.join(build.OBJ, "decode_valu.o")):
        build.build()
    return build_sanitized.build(str(tmp_path_factory.mktemp("san")))


def test_block_manager_traces_are_clean(san):
    r = subprocess.run([san["driver"], "200"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "200 traces, 0 failed checks" in r.stdout


def test_abi_and_block_manager_tests_on_the_instrumented_library(san):
    env = dict(os.environ, PA_LIB=san["lib"], LD_PRELOAD=san["asan_runtime"],
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:"
                            "halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest, paged_kv_cache_78_amd as pa; "
            "assert pa.binding._LIB_PATH.endswith('libpa_san.so'); "
            "sys.exit(pytest.main(['-q', '-m', 'not gpu', '-p', 'no:cacheprovider', "
            "'tests/test_block_manager.py', 'tests/test_abi.py', 'tests/test_zz_no_alloc.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
