"""Build and load ``liboracle.so`` (plain C, gcc, OpenMP).

TEST INFRASTRUCTURE (part of the oracle). Compiled with -O2 and
-ffp-contract=off so every product and sum is a separately rounded IEEE
double operation, as written in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def load_library():
    """liboracle.so (built on first use), or the build ORACLE_LIB names
    (the tests' sanitizer run loads an instrumented build that way)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("ORACLE_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(path)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_matmul.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, dp, i64,
                                   i64, i64, i64, vp, i64]
        lib.orc_matmul.restype = ctypes.c_int
        lib.orc_entries.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64,
                                    vp, vp, i64, dp]
        lib.orc_entries.restype = ctypes.c_int
        lib.orc_matvec.argtypes = [vp, ctypes.c_int, i64, i64, i64, dp, dp]
        lib.orc_matvec.restype = ctypes.c_int
        lib.orc_sum_ranked.argtypes = [dp, i64, ctypes.c_int, i64, dp]
        lib.orc_sum_ranked.restype = ctypes.c_int
        lib.orc_gelu_tanh.argtypes = [ctypes.c_double]
        lib.orc_gelu_tanh.restype = ctypes.c_double
        lib.orc_gelu_tanh_array.argtypes = [dp, dp, i64]
        lib.orc_gelu_tanh_array.restype = ctypes.c_int
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_round_bf16.restype = ctypes.c_uint16
        lib.orc_round_bf16_array.argtypes = [dp, vp, i64]
        lib.orc_round_bf16_array.restype = ctypes.c_int
        _lib = lib
        return lib


if __name__ == "__main__":
    print(build(verbose=True))
