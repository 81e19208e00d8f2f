"""Python access to the C form of the oracle's reduce statistics and bf16
norm tree (test infrastructure only; see oracle_c.c).  Built with gcc by ``build()``."""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle_c.c")


def build() -> str:
    tmp = SO + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
                    SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, SO)
    _lib.cache_clear()
    return SO


@functools.lru_cache(maxsize=None)
def _lib():
    if not os.path.exists(SO):
        build()
    lib = ctypes.CDLL(SO)
    lib.oracle_reduce_stats.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                        ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64),
                                        ctypes.POINTER(ctypes.c_uint64),
                                        ctypes.POINTER(ctypes.c_int32)]
    lib.oracle_reduce_stats.restype = ctypes.c_int
    lib.oracle_reduce_tree_bf16.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                            ctypes.c_int64, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.oracle_reduce_tree_bf16.restype = ctypes.c_int
    return lib


def reduce_stats(rows: np.ndarray, count: int | None = None):
    """rows: [N, >= count] uint16 (fp16 bits), C-contiguous rows.
    Returns (Q, overflow) for the first `count` columns."""
    assert rows.dtype == np.uint16 and rows.ndim == 2 and rows.strides[1] == 2
    n = rows.shape[0]
    count = rows.shape[1] if count is None else count
    ptrs = (ctypes.c_void_p * n)(*[rows[r].ctypes.data for r in range(n)])
    lo, hi, bad = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int32()
    rc = _lib().oracle_reduce_stats(ptrs, n, count, ctypes.byref(lo), ctypes.byref(hi),
                                    ctypes.byref(bad))
    if rc != 0:
        raise ValueError("accumulator outside the exact range")
    return (int(hi.value) << 64) | int(lo.value), bool(bad.value)


def reduce_tree_bf16(rows: np.ndarray, count: int | None = None, width: int | None = None):
    """rows: [N, >= count] uint16 (bf16 bits).  Returns (tree, overflow): the
    pairwise fp64 tree of the exact squares of the first `count` column sums,
    zero-padded to `width` (default: the next power of two)."""
    assert rows.dtype == np.uint16 and rows.ndim == 2 and rows.strides[1] == 2
    n = rows.shape[0]
    count = rows.shape[1] if count is None else count
    if width is None:
        width = 1
        while width < count:
            width *= 2
    ptrs = (ctypes.c_void_p * n)(*[rows[r].ctypes.data for r in range(n)])
    tree, bad = ctypes.c_double(), ctypes.c_int32()
    rc = _lib().oracle_reduce_tree_bf16(ptrs, n, count, width, ctypes.byref(tree),
                                        ctypes.byref(bad))
    if rc != 0:
        raise ValueError("bad width or out of memory")
    return float(tree.value), bool(bad.value)
