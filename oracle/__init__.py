"""CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

The arithmetic lives in ``oracle.cpp`` (plain single-threaded C++, g++); this
module only loads it and marshals numpy arrays.  See that file for the
definitions and the passages of the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

SUM, MAX, MIN = 0, 1, 2


def compile_oracle(src: str, so_path: str) -> str:
    """g++ -> shared library (no HIP involved)."""
    tmp = so_path + ".tmp%d" % os.getpid()
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC",
                           src, "-o", tmp])
    os.replace(tmp, so_path)
    return so_path


def compile_oracle_source(text: str, so_path: str) -> str:
    """Compile C++ source text (tests use this for planted-mistake copies)."""
    src = so_path + ".cpp"
    with open(src, "w") as f:
        f.write(text)
    return compile_oracle(src, so_path)


def build(force: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so if it is missing (or force)."""
    if force or not os.path.exists(_SO):
        compile_oracle(os.path.join(_HERE, "oracle.cpp"), _SO)
    return _SO


class Oracle:
    """ctypes view of one build of oracle.cpp (the default build, or a
    deliberately mutated copy used by the tests to show the pins bite)."""

    def __init__(self, so_path: str):
        lib = ctypes.CDLL(so_path)
        p = ctypes.c_void_p
        lib.oracle_topk_i32.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p]
        lib.oracle_topk_i32.restype = ctypes.c_int
        lib.oracle_reduce_i32.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p]
        lib.oracle_reduce_i32.restype = ctypes.c_int
        lib.oracle_check_topk.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p]
        lib.oracle_check_topk.restype = ctypes.c_int
        lib.oracle_stats_i32.argtypes = [p, ctypes.c_int64, p]
        lib.oracle_stats_i32.restype = ctypes.c_int
        lib.oracle_topk_batched_i32.argtypes = [p, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int32, p]
        lib.oracle_topk_batched_i32.restype = ctypes.c_int
        lib.oracle_topk_merge_i32.argtypes = [p, ctypes.c_int64,
                                              ctypes.c_int32, ctypes.c_int32, p]
        lib.oracle_topk_merge_i32.restype = ctypes.c_int
        lib.oracle_histogram_i32.argtypes = [p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, p]
        lib.oracle_histogram_i32.restype = ctypes.c_int
        lib.oracle_topk_segmented_i32.argtypes = [p, ctypes.c_int64, p,
                                                  ctypes.c_int64,
                                                  ctypes.c_int32, p, p]
        lib.oracle_topk_segmented_i32.restype = ctypes.c_int
        for name in ("oracle_topk_kv_i32", "oracle_topk_kv_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p, p]
            fn.restype = ctypes.c_int
        self.lib = lib

    def topk(self, x, k: int) -> np.ndarray:
        """The k largest values of x, descending (sort-based definition)."""
        a = _as_i32(x)
        out = np.empty(max(k, 0), dtype=np.int32)
        rc = self.lib.oracle_topk_i32(a.ctypes.data, a.size, k,
                                      out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_topk_i32: invalid arguments (n=%d, k=%d)"
                             % (a.size, k))
        return out

    def reduce(self, x, op: int) -> int:
        """Sum (int64), max or min of x; the identity when x is empty."""
        a = _as_i32(x)
        out = np.zeros(1, dtype=np.int64)
        rc = self.lib.oracle_reduce_i32(a.ctypes.data if a.size else None,
                                        a.size, op, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_reduce_i32: invalid arguments (op=%d)"
                             % op)
        return int(out[0])

    def stats(self, x) -> dict:
        """count, sum, max, min and sum of squares of x, as Python ints
        (the sum of squares exact beyond 64 bits)."""
        a = _as_i32(x)
        out = np.zeros(6, dtype=np.int64)
        rc = self.lib.oracle_stats_i32(a.ctypes.data if a.size else None,
                                       a.size, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_stats_i32: invalid arguments")
        u = out.view(np.uint64)
        return {"count": int(out[0]), "sum": int(out[1]), "max": int(out[2]),
                "min": int(out[3]), "sumsq": int(u[4]) | (int(u[5]) << 64)}

    def topk_kv(self, x, k: int):
        """(values, int64 positions) of the k largest elements of x, int32 or
        float32, ordered by value descending, then position ascending."""
        a = np.ascontiguousarray(x)
        if a.ndim != 1 or a.dtype not in (np.int32, np.float32):
            raise ValueError("expected a 1-D int32 or float32 array")
        fn = (self.lib.oracle_topk_kv_i32 if a.dtype == np.int32
              else self.lib.oracle_topk_kv_f32)
        vals = np.empty(max(k, 0), dtype=a.dtype)
        idx = np.empty(max(k, 0), dtype=np.int64)
        rc = fn(a.ctypes.data, a.size, k, vals.ctypes.data, idx.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_topk_kv: invalid arguments (n=%d, k=%d)"
                             % (a.size, k))
        return vals, idx

    def topk_batched(self, x, k: int, cols: int | None = None) -> np.ndarray:
        """Top-k of every row of the 2-D int32 array x, shape (rows, k).
        With cols given, only the first cols columns of each row count
        (the rest is the row stride's padding)."""
        a = np.ascontiguousarray(x, dtype=np.int32)
        if a.ndim != 2:
            raise ValueError("expected a 2-D array")
        rows, ld = a.shape
        c = ld if cols is None else cols
        out = np.empty((rows, max(k, 0)), dtype=np.int32)
        rc = self.lib.oracle_topk_batched_i32(a.ctypes.data, rows, c, ld, k,
                                              out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_topk_batched_i32: invalid arguments "
                             "(rows=%d, cols=%d, ld=%d, k=%d)"
                             % (rows, c, ld, k))
        return out

    def topk_merge(self, lists, k: int) -> np.ndarray:
        """The k largest values of the union of the rows of `lists` (a 2-D
        int32 array whose rows are each in descending order)."""
        a = np.ascontiguousarray(lists, dtype=np.int32)
        if a.ndim != 2:
            raise ValueError("expected a 2-D array")
        m, ln = a.shape
        out = np.empty(max(k, 0), dtype=np.int32)
        rc = self.lib.oracle_topk_merge_i32(a.ctypes.data, m, ln, k,
                                            out.ctypes.data)
        if rc == -2:
            raise ValueError("oracle_topk_merge_i32: a list is not in "
                             "descending order")
        if rc != 0:
            raise ValueError("oracle_topk_merge_i32: invalid arguments "
                             "(m=%d, len=%d, k=%d)" % (m, ln, k))
        return out

    def topk_segmented(self, x, offsets, k: int):
        """(out, counts): the top-k of every segment x[offsets[s] ..
        offsets[s+1]), shape (nseg, k), a short segment's values followed by
        INT32_MIN; counts[s] = min(k, segment length)."""
        a = _as_i32(x)
        off = np.ascontiguousarray(offsets, dtype=np.int64)
        if off.ndim != 1 or off.size < 1:
            raise ValueError("offsets: a 1-D array of nseg + 1 entries")
        nseg = off.size - 1
        out = np.empty((nseg, max(k, 0)), dtype=np.int32)
        counts = np.empty(nseg, dtype=np.int32)
        rc = self.lib.oracle_topk_segmented_i32(
            a.ctypes.data if a.size else None, a.size, off.ctypes.data, nseg,
            k, out.ctypes.data if nseg else None, counts.ctypes.data)
        if rc == -2:
            raise ValueError("oracle_topk_segmented_i32: offsets out of "
                             "order or outside the array")
        if rc != 0:
            raise ValueError("oracle_topk_segmented_i32: invalid arguments "
                             "(n=%d, nseg=%d, k=%d)" % (a.size, nseg, k))
        return out, counts

    def histogram(self, x, lo: int, shift: int, nbins: int) -> np.ndarray:
        """int64 counts of x in nbins bins of width 2**shift from lo."""
        a = _as_i32(x)
        out = np.zeros(max(nbins, 0), dtype=np.int64)
        rc = self.lib.oracle_histogram_i32(a.ctypes.data if a.size else None,
                                           a.size, lo, shift, nbins,
                                           out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_histogram_i32: invalid arguments "
                             "(shift=%d, nbins=%d)" % (shift, nbins))
        return out

    def check_topk(self, x, k: int, cand) -> int:
        """0 if cand is exactly the descending top-k of x, else 1/2/3."""
        a = _as_i32(x)
        c = _as_i32(cand)
        if c.size != k:
            return 1
        rc = self.lib.oracle_check_topk(a.ctypes.data, a.size, k,
                                        c.ctypes.data)
        if rc < 0:
            raise ValueError("oracle_check_topk: invalid arguments")
        return rc


def _as_i32(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.int32)
    if a.ndim != 1:
        raise ValueError("expected a 1-D array")
    return a


def default() -> Oracle:
    global _lib
    if _lib is None:
        build()
        _lib = Oracle(_SO)
    return _lib


def topk(x, k: int) -> np.ndarray:
    return default().topk(x, k)


def reduce(x, op: int) -> int:
    return default().reduce(x, op)


def check_topk(x, k: int, cand) -> int:
    return default().check_topk(x, k, cand)


def stats(x) -> dict:
    return default().stats(x)


def topk_kv(x, k: int):
    return default().topk_kv(x, k)


def histogram(x, lo: int, shift: int, nbins: int) -> np.ndarray:
    return default().histogram(x, lo, shift, nbins)


def topk_batched(x, k: int, cols: int | None = None) -> np.ndarray:
    return default().topk_batched(x, k, cols)


def topk_merge(lists, k: int) -> np.ndarray:
    return default().topk_merge(lists, k)


def topk_segmented(x, offsets, k: int):
    return default().topk_segmented(x, offsets, k)
