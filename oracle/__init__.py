"""CPU oracle for the exact row-wise bf16 top-k -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it shares no code with that library.

The arithmetic lives in ``tk_oracle.c`` (plain C, built with gcc and no
fast-math): widen every bf16 to double, drop NaN, sort by value descending and
column ascending, keep the first k.  This module only builds and loads that
library and marshals numpy arrays into it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tk_oracle.c")
LIBRARY = os.path.join(_HERE, "libtk_oracle.so")

FILL_IDX = -1
FILL_VAL = 0x7FC0
MASK_NAN, MASK_POSINF, MASK_NEGINF = 1, 2, 4


def build_command(source: str = SOURCE, output: str = LIBRARY) -> list[str]:
    return ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", source, "-o", output, "-lm"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = output + ".tmp"
    subprocess.run(build_command(source, tmp), check=True)
    os.replace(tmp, output)
    return output


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the oracle library, compiling it first only if it is not built."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != LIBRARY:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    for name in ("tko_topk_bf16", "tko_topk_f16"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    f = lib.tko_topk_f32
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    for name in ("tko_bf16_value", "tko_f16_value"):
        f = getattr(lib, name)
        f.restype = ctypes.c_double
        f.argtypes = [ctypes.c_uint16]
    _lib_cache[path] = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def topk_bf16(m: np.ndarray, cols: int, k: int, threads: int | None = None, lib: ctypes.CDLL | None = None):
    """Top-k of every row of a (rows, stride) uint16 bf16 matrix over columns [0, cols).

    Returns (idx int32 [rows,k], val uint16 [rows,k], count int32 [rows], mask uint32 [rows]).
    """
    return _topk("tko_topk_bf16", m, cols, k, threads, lib)


def topk_f16(m: np.ndarray, cols: int, k: int, threads: int | None = None, lib: ctypes.CDLL | None = None):
    """The same for a matrix of IEEE fp16 bit patterns."""
    return _topk("tko_topk_f16", m, cols, k, threads, lib)


def topk_f32(m: np.ndarray, cols: int, k: int, threads: int | None = None, lib: ctypes.CDLL | None = None):
    """Top-k of every row of a (rows, stride) uint32 matrix of fp32 bit patterns.

    Returns (idx int32 [rows,k], val uint32 [rows,k] fp32 bits, count int32 [rows], mask uint32 [rows]).
    """
    m = np.ascontiguousarray(m, dtype=np.uint32)
    assert m.ndim == 2 and cols <= m.shape[1]
    rows, stride = m.shape
    lib = lib or load()
    idx = np.empty((rows, k), dtype=np.int32)
    val = np.empty((rows, k), dtype=np.uint32)
    cnt = np.empty(rows, dtype=np.int32)
    mask = np.empty(rows, dtype=np.uint32)
    t = default_threads() if threads is None else threads
    rc = lib.tko_topk_f32(rows, cols, stride, k, m.ctypes.data, idx.ctypes.data, val.ctypes.data, cnt.ctypes.data,
                          mask.ctypes.data, t)
    if rc != 0:
        raise RuntimeError(f"oracle failed (rc={rc}) rows={rows} cols={cols} stride={stride} k={k}")
    return idx, val, cnt, mask


def _topk(fn: str, m, cols, k, threads, lib):
    m = np.ascontiguousarray(m, dtype=np.uint16)
    assert m.ndim == 2 and cols <= m.shape[1]
    rows, stride = m.shape
    lib = lib or load()
    idx = np.empty((rows, k), dtype=np.int32)
    val = np.empty((rows, k), dtype=np.uint16)
    cnt = np.empty(rows, dtype=np.int32)
    mask = np.empty(rows, dtype=np.uint32)
    t = default_threads() if threads is None else threads
    rc = getattr(lib, fn)(rows, cols, stride, k, m.ctypes.data, idx.ctypes.data, val.ctypes.data,
                          cnt.ctypes.data, mask.ctypes.data, t)
    if rc != 0:
        raise RuntimeError(f"oracle failed (rc={rc}) rows={rows} cols={cols} stride={stride} k={k}")
    return idx, val, cnt, mask
