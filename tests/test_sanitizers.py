"""CPU: the oracle and the C ABI's host code (argument validation, workspace
sizing, chunking, launch order) under the address and undefined-behaviour
sanitizers.  tests/sanitize/build_sanitized.py builds both (the ABI's kernels
replaced by host stubs); the oracle pins and the ABI tests then run in a
subprocess with the sanitizer runtime preloaded, and any report aborts it."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))
import build_sanitized  # noqa: E402

ORACLE_TESTS = ["test_oracle_pins.py", "test_oracle_mask_modes.py", "test_oracle_options.py",
                "test_oracle_bwd_pins.py"]


def instrumented(path):
    syms = subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout
    return "__asan_report" in syms and "__ubsan_handle" in syms


def run_suite(files, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4", **env_extra)
    # the child prints which library it loaded, then runs the tests
    code = ("import sys, pytest; sys.path.insert(0, %r); " % os.path.dirname(HERE) +
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + %r))" %
            [os.path.join(HERE, f) for f in files])
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("sanitized"))
    return build_sanitized.build_oracle(d), build_sanitized.build_abi(d), build_sanitized.runtimes()


def test_oracle_under_sanitizers(builds):
    lib, _, (gcc_rt, _) = builds
    assert instrumented(lib)
    out = run_suite(ORACLE_TESTS, {"SA_ORACLE_LIB": lib, "LD_PRELOAD": ":".join(gcc_rt)})
    assert " passed" in out


def test_abi_host_code_under_sanitizers(builds):
    _, lib, (_, clang_rt) = builds
    if clang_rt is None:
        pytest.skip("clang sanitizer runtime not found")
    assert instrumented(lib)
    out = run_suite(["test_library_abi.py"], {"SPARSE_ATTN_LIB": lib, "LD_PRELOAD": clang_rt})
    assert " passed" in out
