"""Python access to the C form of the oracle (test infrastructure only; see
oracle_c.c): the reduce statistics, the bf16 norm tree, and the element-wise
rest of the step (unscale, Adam, 16-bit cast) for whole-shard comparisons.
Built with gcc by ``build()``."""
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
    lib.oracle_cast16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    lib.oracle_cast16.restype = None
    lib.oracle_reduce_unscale.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                          ctypes.c_void_p]
    lib.oracle_reduce_unscale.restype = None
    lib.oracle_adam_update.argtypes = [ctypes.c_void_p] * 5 + [
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int]
    lib.oracle_adam_update.restype = None
    lib.oracle_count_unequal.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int]
    lib.oracle_count_unequal.restype = ctypes.c_int64
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


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def cast16(x: np.ndarray, bf16: bool = False) -> np.ndarray:
    """fp32 -> fp16 (or bf16) bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    _lib().oracle_cast16(_ptr(x), _ptr(out), x.size, 1 if bf16 else 0)
    return out.reshape(x.shape)


def reduce_unscale(rows: np.ndarray, inv32, count: int | None = None, bf16: bool = False,
                   out: np.ndarray | None = None) -> np.ndarray:
    """g = f32(acc * inv32) for the first `count` columns of rows ([N, >= count]
    uint16 fp16 or bf16 bits), acc the rank-ordered fp32 sum from +0."""
    assert rows.dtype == np.uint16 and rows.ndim == 2 and rows.strides[1] == 2
    n = rows.shape[0]
    count = rows.shape[1] if count is None else count
    g = np.empty(count, dtype=np.float32) if out is None else out
    assert g.dtype == np.float32 and g.size >= count and g.flags["C_CONTIGUOUS"]
    ptrs = (ctypes.c_void_p * n)(*[rows[r].ctypes.data for r in range(n)])
    _lib().oracle_reduce_unscale(ptrs, n, count, 1 if bf16 else 0, float(np.float32(inv32)),
                                 _ptr(g))
    return g


def adam_update(g, p, m, v, slot, sc, coef, bf16: bool = False):
    """In place on p, m, v (fp32) and slot (uint16): the oracle's adam_apply
    with the Scalars `sc` and clip coefficient `coef`, and the 16-bit cast."""
    n = g.size
    for a, dt in ((g, np.float32), (p, np.float32), (m, np.float32), (v, np.float32),
                  (slot, np.uint16)):
        assert a.dtype == dt and a.size == n and a.flags["C_CONTIGUOUS"]
    scal = np.array([sc.b1, sc.omb1, sc.b2, sc.omb2, sc.eps, sc.step_size, sc.sqrt_bc2,
                     sc.decay], dtype=np.float32)
    _lib().oracle_adam_update(_ptr(g), _ptr(p), _ptr(m), _ptr(v), _ptr(slot), n, _ptr(scal),
                              float(np.float32(coef)), 1 if bf16 else 0)


def count_unequal(a: np.ndarray, b: np.ndarray) -> int:
    """Positions where two equal-length arrays of 2- or 4-byte words differ bitwise."""
    assert a.itemsize == b.itemsize and a.size == b.size
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return int(_lib().oracle_count_unequal(_ptr(a), _ptr(b), a.size, a.itemsize))
