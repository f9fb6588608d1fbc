"""ctypes access to liboracle.so (the fp64 C part of the oracle).  Test infrastructure only."""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "medusa_oracle.c")
# MEDUSA_ORACLE_LIB names another build of the same source (the sanitizer test's), used as is
LIB = os.environ.get("MEDUSA_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1}

_lib = None


def build(force=True):
    """Compile liboracle.so with gcc: -O2, no fast-math, OpenMP over independent units."""
    if force or not os.path.exists(LIB):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o",
                               LIB + ".tmp", SRC, "-lm"])
        os.replace(LIB + ".tmp", LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            if os.environ.get("MEDUSA_ORACLE_LIB"):
                raise FileNotFoundError(LIB)
            build()
        L = ctypes.CDLL(LIB)
        vp, dp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
        L.oracle_project.argtypes = [vp, ctypes.c_int, ctypes.c_long, ctypes.c_int, dp,
                                     ctypes.c_long, ctypes.c_int, dp, ctypes.c_long]
        L.oracle_heads.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_long, ctypes.c_int, dp, dp]
        L.oracle_topk.argtypes = [dp, ctypes.c_long, ctypes.c_long, ctypes.c_int, ip, dp]
        L.oracle_tree_attention.argtypes = [vp, vp, vp, ctypes.c_int, ip, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_long, ip, ctypes.c_int,
                                            ctypes.c_double, ip, ctypes.c_long, dp]
        for f in (L.oracle_project, L.oracle_heads, L.oracle_topk, L.oracle_tree_attention):
            f.restype = None
        _lib = L
    return _lib


def vptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def check_input(a, dtype):
    want = np.float32 if dtype == "f32" else np.uint16
    assert a.dtype == want, (a.dtype, dtype)
    assert a.flags.c_contiguous
    return a


def set_threads(n):
    """Threads the OpenMP loops of the C part use from now on (for timing the oracle; its results
    do not depend on it: every sum keeps its order).  Returns the count now in force."""
    L = lib()
    L.omp_set_num_threads(int(n))
    L.omp_get_max_threads.restype = ctypes.c_int
    return int(L.omp_get_max_threads())
