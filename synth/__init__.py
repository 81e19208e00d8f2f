"""Seeded synthetic inputs shared by the CPU oracle and the GPU feeder.

Holds no step of the method.  Every value comes from ``libsynth.so`` (built
from ``synth.c``), so the oracle and the device path see the same bits.

Stream layout (Philox4x32-10, key = (BASE_SEED, workload id)):
  counter = (block lo, block hi, word2, word3) with element e in block e // 4,
  word2 = contributing rank (contributions) or 0,
  word3 = purpose << 24 | step.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

from .workloads import (  # noqa: F401
    ALL, BF16_WORKLOADS, BY_NAME, FLAT75, GPT2, GPT2_FSDP, LLAMA2_70B, LLAMA3_8B,
    LLAMA3_8B_BF16, LLAMA3_8B_FSDP, PURPOSE_CONTRIB, PURPOSE_INJECT, PURPOSE_MASTER, TINY,
    TINY_BF16, TINY_FSDP, UNIT_WORKLOADS, Workload,
)

FORMATS = {"fp16": 0, "bf16": 1}
PLUS_INF = {"fp16": 0x7C00, "bf16": 0x7F80}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")


def build() -> str:
    """Compile libsynth.so with gcc (OpenMP, no FP contraction)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    _lib.cache_clear()
    return _SO


@functools.lru_cache(maxsize=None)
def _lib() -> ctypes.CDLL:
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u32, i64 = ctypes.c_uint32, ctypes.c_int64
    vp = ctypes.c_void_p
    lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
    lib.synth_fp16_table_size.restype = i64
    lib.synth_table_size.argtypes = [ctypes.c_int]
    lib.synth_table_size.restype = i64
    lib.synth_normal_table.argtypes = [ctypes.c_int, ctypes.c_double, vp, vp, vp]
    lib.synth_normal_table.restype = ctypes.c_int
    lib.synth_fp16_normal.argtypes = [u32, u32, u32, u32, i64, i64, i64, vp, vp, vp, vp]
    lib.synth_f32_normal.argtypes = [u32, u32, u32, u32, i64, i64, i64, ctypes.c_double, vp]
    lib.synth_words.argtypes = [u32, u32, u32, u32, i64, i64, vp]
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def philox4x32_10(ctr, key) -> Tuple[int, int, int, int]:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    _lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return tuple(int(x) for x in o)


@functools.lru_cache(maxsize=16)
def normal_table(std: float, fmt: str = "fp16"):
    """(thresholds uint64, bit patterns uint16, guide uint32) for N(0, std^2)
    on the grid of fmt ("fp16" or "bf16")."""
    f = FORMATS[fmt]
    n = int(_lib().synth_table_size(f))
    thr = np.zeros(n, dtype=np.uint64)
    val = np.zeros(n, dtype=np.uint16)
    guide = np.zeros(65536, dtype=np.uint32)
    rc = _lib().synth_normal_table(f, float(std), _ptr(thr), _ptr(val), _ptr(guide))
    if rc != 0:
        raise ValueError(f"bad table std {std}")
    for a in (thr, val, guide):
        a.setflags(write=False)
    return thr, val, guide


def fp16_normal_table(std: float):
    return normal_table(std, "fp16")


def contributions(w: Workload, step: int, rank: int, begin: int, count: int, loss_scale: float,
                  out: Optional[np.ndarray] = None) -> np.ndarray:
    """Bit patterns (fp16 or bf16, per the workload) of rank ``rank``'s scaled
    gradient at flat elements [begin, begin+count) for 1-based step ``step``:
    N(0, (sigma*loss_scale)^2) on the format's grid; elements at or past psi
    are +0 (padding).  Includes the workload's injected +inf, if any."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size >= count
    thr, val, guide = normal_table(w.sigma * loss_scale, w.dtype)
    _lib().synth_fp16_normal(w.key[0], w.key[1], rank, (PURPOSE_CONTRIB << 24) | step, begin, count,
                             w.psi, _ptr(thr), _ptr(val), _ptr(guide), _ptr(out))
    site = inject_site(w, step)
    if site is not None:
        q, e = site
        if q == rank and begin <= e < begin + count:
            out[e - begin] = PLUS_INF[w.dtype]
    return out


def masters(w: Workload, begin: int, count: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Initial fp32 master weights at flat elements [begin, begin+count):
    f32(master_sigma * z); +0 past psi."""
    if out is None:
        out = np.empty(count, dtype=np.float32)
    assert out.dtype == np.float32 and out.size >= count
    _lib().synth_f32_normal(w.key[0], w.key[1], 0, PURPOSE_MASTER << 24, begin, count, w.psi,
                            float(w.master_sigma), _ptr(out))
    return out


def words(w: Workload, word2: int, word3: int, begin: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint32)
    _lib().synth_words(w.key[0], w.key[1], word2, word3, begin, count, _ptr(out))
    return out


def inject_site(w: Workload, step: int) -> Optional[Tuple[int, int]]:
    """(contributing rank q, flat element e) of the one +inf injected at
    ``step``, or None.  e < psi // N, which lies in rank 0's shard under any
    partition whose first shard holds at least psi / N elements."""
    if w.inject_step is None or step != w.inject_step:
        return None
    n = w.world_size
    x = words(w, 0, (PURPOSE_INJECT << 24) | step, 0, 4)
    q = int(x[0]) % n
    e = ((int(x[1]) << 32) | int(x[2])) % (w.psi // n)
    return q, e
