"""Seeded synthetic int32 inputs shared by the CPU oracle side and the GPU side.

The arrays are produced by ``gen.c`` (SplitMix64 used counter-style; see that
file for the exact definition).  This module holds none of the arithmetic of
the method under test: top-k and reductions live in ``oracle/`` (CPU, test
infrastructure) and in the HIP library (GPU), which share no code.

Workloads, named by what they are (values, distribution, size):

==========================  ===========  ==========================  ====
name                        n            values                      seed
==========================  ===========  ==========================  ====
``full_1e6``                1,000,000    uniform over all of int32     1
``pm1000_2p26``             2**26        uniform over [-1000, 1000]    2
``full_1e8``                100,000,000  uniform over all of int32     3
``dup1000_1e7``             10,000,000   uniform over [0, 1000)        4
``full_1e9``                1e9          uniform over all of int32     5
==========================  ===========  ==========================  ====

``dup1000_1e7`` also comes in two variants: ``sorted`` (the same values in
ascending order, the worst case for insertion-based selection) and ``equal``
(n copies of the draw's element 0).

``segment_offsets`` cuts an array into segments of varied lengths (the
segmented top-k's input): lengths drawn log-uniformly from [lo, hi] with
numpy's PCG64 generator under a fixed seed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

WORKLOADS = {
    "full_1e6": dict(n=1_000_000, lo=0, range=0, seed=1),
    "pm1000_2p26": dict(n=1 << 26, lo=-1000, range=2001, seed=2),
    "full_1e8": dict(n=100_000_000, lo=0, range=0, seed=3),
    "dup1000_1e7": dict(n=10_000_000, lo=0, range=1000, seed=4),
    "full_1e9": dict(n=1_000_000_000, lo=0, range=0, seed=5),
}


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (plain gcc, host only)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "gen.c")
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC",
                               "-pthread", src, "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        lib.synth_fill_i32.argtypes = [ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.c_int]
        lib.synth_fill_i32.restype = ctypes.c_int
        lib.synth_raw_u64.argtypes = [ctypes.c_uint64, ctypes.c_int64]
        lib.synth_raw_u64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill(seed: int, n: int, lo: int = 0, range_: int = 0) -> np.ndarray:
    """n int32 values: full int32 range if range_ == 0, else [lo, lo+range_)."""
    if n < 0:
        raise ValueError("n must be >= 0")
    if not (0 <= range_ < 2**32):
        raise ValueError("range_ must be in [0, 2**32)")
    out = np.empty(n, dtype=np.int32)
    rc = _load().synth_fill_i32(seed, n, lo, range_,
                                out.ctypes.data if n else None, _threads())
    if rc != 0:
        raise RuntimeError("synth_fill_i32 failed")
    return out


def raw_u64(seed: int, i: int) -> int:
    """The 64-bit SplitMix64 output behind element i."""
    return int(_load().synth_raw_u64(seed, i))


def workload(name: str, variant: str | None = None, n: int | None = None,
             seed: int | None = None) -> np.ndarray:
    """Materialise a named workload (optionally truncated to n elements).

    variant: None, "sorted" (ascending) or "equal" (n copies of element 0).
    """
    spec = WORKLOADS[name]
    size = spec["n"] if n is None else n
    s = spec["seed"] if seed is None else seed
    x = fill(s, size, spec["lo"], spec["range"])
    if variant is None:
        return x
    if variant == "sorted":
        x.sort(kind="stable")
        return x
    if variant == "equal":
        if size:
            x[:] = x[0]
        return x
    raise ValueError("unknown variant %r" % variant)


def segment_offsets(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """int64 offsets (nseg + 1 entries, from 0 to n) cutting n elements into
    consecutive segments whose lengths are drawn log-uniformly from
    [lo, hi] (rounded down), the last one cut short at n."""
    if not (1 <= lo <= hi) or n < 0:
        raise ValueError("need 1 <= lo <= hi and n >= 0")
    rng = np.random.default_rng(seed)
    out = [0]
    pos = 0
    while pos < n:
        chunk = rng.random(4096)
        lens = np.floor(np.exp(np.log(lo) + chunk * (np.log(hi + 1) -
                                                      np.log(lo))))
        for ln in np.clip(lens, lo, hi).astype(np.int64):
            pos = min(n, pos + int(ln))
            out.append(pos)
            if pos >= n:
                break
    return np.asarray(out, dtype=np.int64)
