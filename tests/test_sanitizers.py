"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host planner (plan.cpp: parsing of caller-supplied spec text,
the four-case classification, shapes and offsets from caller sizes) and the
oracle's C loops (oracle.c) are built with gcc's sanitizers, and a child
Python process loads those builds (SHARDMM_LIB, ORACLE_LIB) with the
sanitizer runtimes preloaded, then runs the planner brute force against the
oracle planner, the host-call tests and the oracle pins. Any sanitizer
report aborts the child, and the test fails with its output. The device
entry points are not part of these builds (their host checks run in the
ordinary CPU tests; GPU code is not sanitized here).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "local_shard_gemm_amd")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

# host-call tests of the library (no device entry point involved)
HOST_TESTS = ("parse_spec or mesh_errors or planner_brute_force or case4_extreme or sandbox_default or "
              "plan_dtype_rules or gathered_plan_examples or mesh_rank_limit or status_strings or "
              "plan_struct_layout")


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    out = tmp_path_factory.mktemp("san")
    plan_lib = str(out / "libshardmm_plan_san.so")
    oracle_lib = str(out / "liboracle_san.so")
    subprocess.run(["g++", "-std=c++17", *SAN, "-fPIC", "-shared", "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(PKG, "csrc"), os.path.join(PKG, "csrc", "plan.cpp"), "-o", plan_lib],
                   check=True)
    subprocess.run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_lib, "-lm"], check=True)
    env = dict(os.environ)
    env.update({
        "SHARDMM_LIB": plan_lib,
        "ORACLE_LIB": oracle_lib,
        "LD_PRELOAD": " ".join([_runtime("libasan.so"), _runtime("libubsan.so")]),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    return env


def _run(env, *args):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_planner_under_sanitizers(sanitized):
    """The library's planner on every spec pair of the brute force, the
    extreme shapes and every parse and error path, instrumented."""
    out = _run(sanitized, "tests/test_abi_cpu.py", "-k", HOST_TESTS)
    assert " passed" in out


def test_oracle_under_sanitizers(sanitized):
    """The oracle's loops under the pins and the planner cases, instrumented."""
    out = _run(sanitized, "tests/test_oracle_pins.py", "tests/test_oracle_planner.py")
    assert " passed" in out
