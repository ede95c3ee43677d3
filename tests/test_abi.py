"""The C-ABI library: it loads, exports every entry point include/libtopk.h
declares, and rejects invalid arguments before touching the GPU.  Runs on the
CPU; no compute call reaches a device here."""
import ctypes
import os
import re

import pytest

import top_selection_two_amd as ltk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libtopk.h")
FAKE = 0x10000  # a 64 KiB-aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;",
                       text, flags=re.M)
    return sorted(set(names))


def no_gpu():
    if os.path.exists("/dev/kfd"):
        return False
    import torch
    return torch.cuda.device_count() == 0


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"topk_i32", "reduce_i32", "reduce_stats_i32", "topk_kv_i32",
            "topk_kv_f32", "topk_batched_i32", "topk_merge_i32",
            "histogram_i32",
            "libtopk_strerror",
            "libtopk_max_k", "libtopk_set_grid", "libtopk_grid_for",
            "libtopk_release"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ltk.LIBRARY_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(ltk.SIGNATURES)


def test_constants_match_header():
    text = open(HEADER).read()
    for name, val in [("LIBTOPK_OK", 0), ("LIBTOPK_ERR_INVALID", 1),
                      ("LIBTOPK_ERR_UNSUPPORTED", 2), ("LIBTOPK_ERR_NOMEM", 3),
                      ("LIBTOPK_ERR_HIP", 4), ("LIBTOPK_SUM", 0),
                      ("LIBTOPK_MAX", 1), ("LIBTOPK_MIN", 2)]:
        assert re.search(r"\b%s\s*=\s*%d\b" % (name, val), text), name
    assert re.search(r"#define LIBTOPK_MAX_K 128\b", text)
    assert re.search(r"#define LIBTOPK_MAX_K_SELECT %d\b" % ltk.MAX_K_SELECT,
                     text)
    assert re.search(r"#define LIBTOPK_MAX_BINS %d\b" % ltk.MAX_BINS, text)
    assert ltk.max_k() == 128


def test_strerror():
    for s in range(5):
        assert ltk.strerror(s)
    assert ltk.strerror(99) == "unknown status"
    assert ltk.strerror(0) == "success"


@pytest.mark.parametrize("args,status", [
    ((0, 100, 5, FAKE), ltk.ERR_INVALID),                  # NULL input
    ((FAKE, 100, 5, 0), ltk.ERR_INVALID),                  # NULL output
    ((FAKE + 2, 100, 5, FAKE * 4), ltk.ERR_INVALID),       # misaligned input
    ((FAKE, 100, 5, FAKE * 4 + 1), ltk.ERR_INVALID),       # misaligned output
    ((FAKE, 0, 1, FAKE * 4), ltk.ERR_INVALID),             # n = 0
    ((FAKE, -5, 1, FAKE * 4), ltk.ERR_INVALID),            # n < 0
    ((FAKE, (1 << 32) + 1, 5, 1 << 40), ltk.ERR_INVALID),  # n > 2^32
    ((FAKE, 100, 0, FAKE * 4), ltk.ERR_INVALID),           # k = 0
    ((FAKE, 100, -3, FAKE * 4), ltk.ERR_INVALID),          # k < 0
    ((FAKE, 10, 11, FAKE * 4), ltk.ERR_INVALID),           # k > n
    ((FAKE, 100000, 16385, FAKE * 64), ltk.ERR_UNSUPPORTED),  # k above max
    ((FAKE, 1000, 20, FAKE + 400), ltk.ERR_INVALID),       # out inside in
    ((FAKE, 1000, 20, FAKE - 40), ltk.ERR_INVALID),        # out overlaps in
])
def test_topk_rejects_invalid_arguments(args, status):
    assert ltk.topk_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, 100, 5, FAKE), ltk.ERR_INVALID),                  # NULL input
    ((FAKE, 100, 5, 0), ltk.ERR_INVALID),                  # NULL output
    ((FAKE + 2, 100, 5, FAKE * 4), ltk.ERR_INVALID),       # misaligned input
    ((FAKE, 0, 1, FAKE * 4), ltk.ERR_INVALID),             # n = 0
    ((FAKE, (1 << 32) + 1, 5, 1 << 40), ltk.ERR_INVALID),  # n > 2^32
    ((FAKE, 100, 0, FAKE * 4), ltk.ERR_INVALID),           # k = 0
    ((FAKE, 10, 11, FAKE * 4), ltk.ERR_INVALID),           # k > n
    ((FAKE, 1000, 129, FAKE * 64), ltk.ERR_UNSUPPORTED),   # beyond the array
    ((FAKE, 1000, 20, FAKE + 400), ltk.ERR_INVALID),       # out inside in
])
def test_topk_noalloc_rejects_invalid_arguments(args, status):
    assert ltk.topk_noalloc_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 10, 0, 0), ltk.ERR_INVALID),                   # NULL output
    ((FAKE, 10, 0, FAKE * 4 + 4), ltk.ERR_INVALID),        # misaligned output
    ((FAKE + 1, 10, 0, FAKE * 4), ltk.ERR_INVALID),        # misaligned input
    ((0, 10, 0, FAKE * 4), ltk.ERR_INVALID),               # NULL input, n > 0
    ((FAKE, -1, 0, FAKE * 4), ltk.ERR_INVALID),            # n < 0
    ((FAKE, (1 << 32) + 1, 0, 1 << 40), ltk.ERR_INVALID),  # n > 2^32
    ((FAKE, 10, 3, FAKE * 4), ltk.ERR_INVALID),            # unknown op
    ((FAKE, 10, -1, FAKE * 4), ltk.ERR_INVALID),           # unknown op
    ((FAKE, 10, 0, FAKE + 8), ltk.ERR_INVALID),            # out inside in
])
def test_reduce_rejects_invalid_arguments(args, status):
    assert ltk.reduce_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 10, 0), ltk.ERR_INVALID),                      # NULL output
    ((FAKE, 10, FAKE * 4 + 4), ltk.ERR_INVALID),           # out not 8-aligned
    ((FAKE + 1, 10, FAKE * 4), ltk.ERR_INVALID),           # misaligned input
    ((0, 10, FAKE * 4), ltk.ERR_INVALID),                  # NULL input, n > 0
    ((FAKE, -1, FAKE * 4), ltk.ERR_INVALID),               # n < 0
    ((FAKE, (1 << 32) + 1, 1 << 40), ltk.ERR_INVALID),     # n > 2^32
    ((FAKE, 100, FAKE + 16), ltk.ERR_INVALID),             # out inside in
    ((FAKE, 100, FAKE - 24), ltk.ERR_INVALID),             # out overlaps in
])
def test_stats_rejects_invalid_arguments(args, status):
    assert ltk.stats_raw(*args) == status


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("args,status", [
    ((0, 100, 5, FAKE * 4, FAKE * 8), ltk.ERR_INVALID),          # NULL input
    ((FAKE, 100, 5, 0, FAKE * 8), ltk.ERR_INVALID),              # NULL values
    ((FAKE, 100, 5, FAKE * 4, 0), ltk.ERR_INVALID),              # NULL indices
    ((FAKE + 2, 100, 5, FAKE * 4, FAKE * 8), ltk.ERR_INVALID),   # misaligned in
    ((FAKE, 100, 5, FAKE * 4 + 1, FAKE * 8), ltk.ERR_INVALID),   # misaligned vals
    ((FAKE, 100, 5, FAKE * 4, FAKE * 8 + 4), ltk.ERR_INVALID),   # indices not 8-aligned
    ((FAKE, 0, 1, FAKE * 4, FAKE * 8), ltk.ERR_INVALID),         # n = 0
    ((FAKE, 1 << 32, 5, 1 << 40, 1 << 41), ltk.ERR_INVALID),     # n = 2^32
    ((FAKE, 100, 0, FAKE * 4, FAKE * 8), ltk.ERR_INVALID),       # k = 0
    ((FAKE, 10, 11, FAKE * 4, FAKE * 8), ltk.ERR_INVALID),       # k > n
    ((FAKE, 1000, 129, FAKE * 4, FAKE * 8), ltk.ERR_UNSUPPORTED),
    ((FAKE, 1000, 20, FAKE + 400, FAKE * 8), ltk.ERR_INVALID),   # vals inside in
    ((FAKE, 1000, 20, FAKE * 4, FAKE + 800), ltk.ERR_INVALID),   # indices inside in
    ((FAKE, 100, 20, FAKE * 8, FAKE * 8 + 40), ltk.ERR_INVALID), # vals/indices overlap
])
def test_topk_kv_rejects_invalid_arguments(args, status, f32):
    assert ltk.topk_kv_raw(*args, f32=f32) == status


@pytest.mark.parametrize("args,status", [
    # (in, rows, cols, ld, k, out)
    ((0, 4, 100, 100, 5, FAKE * 64), ltk.ERR_INVALID),           # NULL input
    ((FAKE, 4, 100, 100, 5, 0), ltk.ERR_INVALID),                # NULL output
    ((FAKE + 2, 4, 100, 100, 5, FAKE * 64), ltk.ERR_INVALID),    # misaligned in
    ((FAKE, 4, 100, 100, 5, FAKE * 64 + 2), ltk.ERR_INVALID),    # misaligned out
    ((FAKE, -1, 100, 100, 5, FAKE * 64), ltk.ERR_INVALID),       # rows < 0
    ((FAKE, 4, 0, 100, 1, FAKE * 64), ltk.ERR_INVALID),          # cols = 0
    ((FAKE, 4, (1 << 32) + 1, 1 << 33, 5, 1 << 46), ltk.ERR_INVALID),  # cols
    ((FAKE, 4, 100, 99, 5, FAKE * 64), ltk.ERR_INVALID),         # ld < cols
    ((FAKE, 4, 100, 100, 0, FAKE * 64), ltk.ERR_INVALID),        # k = 0
    ((FAKE, 4, 10, 10, 11, FAKE * 64), ltk.ERR_INVALID),         # k > cols
    ((FAKE, 4, 1000, 1000, 129, FAKE * 64), ltk.ERR_UNSUPPORTED),
    ((FAKE, 1 << 40, 1 << 30, 1 << 30, 5, FAKE * 64), ltk.ERR_INVALID),  # span
    ((FAKE, 4, 100, 100, 5, FAKE + 800), ltk.ERR_INVALID),       # out inside in
    ((FAKE, 4, 100, 1000, 5, FAKE + 4 * 3000), ltk.ERR_INVALID), # out in a gap
    ((FAKE, 4, 100, 100, 20, FAKE - 40), ltk.ERR_INVALID),       # out overlaps
])
def test_topk_batched_rejects_invalid_arguments(args, status):
    assert ltk.topk_batched_raw(*args) == status


def test_topk_batched_zero_rows_is_a_no_op():
    # Validated, nothing enqueued: no device is needed.
    assert ltk.topk_batched_raw(FAKE, 0, 100, 100, 5, FAKE * 64) == ltk.OK
    assert ltk.topk_batched_raw(0, 0, 100, 100, 5, 0) == ltk.OK
    assert ltk.topk_batched_raw(0, 0, 100, 100, 101, 0) == ltk.ERR_INVALID


@pytest.mark.parametrize("args,status", [
    # (lists, m, len, k, out)
    ((0, 8, 20, 20, FAKE * 64), ltk.ERR_INVALID),                # NULL lists
    ((FAKE, 8, 20, 20, 0), ltk.ERR_INVALID),                     # NULL output
    ((FAKE + 1, 8, 20, 20, FAKE * 64), ltk.ERR_INVALID),         # misaligned
    ((FAKE, 8, 20, 20, FAKE * 64 + 3), ltk.ERR_INVALID),         # misaligned
    ((FAKE, 0, 20, 1, FAKE * 64), ltk.ERR_INVALID),              # m = 0
    ((FAKE, (1 << 20) + 1, 1, 1, FAKE * 64), ltk.ERR_INVALID),   # m > 2^20
    ((FAKE, 8, 0, 1, FAKE * 64), ltk.ERR_INVALID),               # len = 0
    ((FAKE, 8, 20, 0, FAKE * 64), ltk.ERR_INVALID),              # k = 0
    ((FAKE, 2, 3, 7, FAKE * 64), ltk.ERR_INVALID),               # k > m * len
    ((FAKE, 8, 200, 129, FAKE * 64), ltk.ERR_UNSUPPORTED),
    ((FAKE, 8, 20, 20, FAKE + 100), ltk.ERR_INVALID),            # out inside
])
def test_topk_merge_rejects_invalid_arguments(args, status):
    assert ltk.topk_merge_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    # (in, n, lo, shift, nbins, out)
    ((FAKE, 100, 0, 0, 16, 0), ltk.ERR_INVALID),                 # NULL output
    ((FAKE, 100, 0, 0, 16, FAKE * 64 + 4), ltk.ERR_INVALID),     # out not 8-aligned
    ((FAKE + 2, 100, 0, 0, 16, FAKE * 64), ltk.ERR_INVALID),     # misaligned in
    ((0, 100, 0, 0, 16, FAKE * 64), ltk.ERR_INVALID),            # NULL in, n > 0
    ((FAKE, -1, 0, 0, 16, FAKE * 64), ltk.ERR_INVALID),          # n < 0
    ((FAKE, (1 << 32) + 1, 0, 0, 16, 1 << 40), ltk.ERR_INVALID), # n > 2^32
    ((FAKE, 100, 0, -1, 16, FAKE * 64), ltk.ERR_INVALID),        # shift < 0
    ((FAKE, 100, 0, 32, 16, FAKE * 64), ltk.ERR_INVALID),        # shift > 31
    ((FAKE, 100, 0, 0, 0, FAKE * 64), ltk.ERR_INVALID),          # nbins = 0
    ((FAKE, 100, 0, 0, 4097, FAKE * 64), ltk.ERR_INVALID),       # nbins > max
    ((FAKE, 100, 0, 0, 16, FAKE + 64), ltk.ERR_INVALID),         # out inside in
])
def test_histogram_rejects_invalid_arguments(args, status):
    assert ltk.histogram_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    # (in, n, offsets, nseg, k, out, counts)
    ((FAKE, 100, FAKE * 8, -1, 5, FAKE * 64, 0), ltk.ERR_INVALID),   # nseg < 0
    ((FAKE, -1, FAKE * 8, 2, 5, FAKE * 64, 0), ltk.ERR_INVALID),     # n < 0
    ((FAKE, (1 << 32) + 1, FAKE * 8, 2, 5, 1 << 40, 0), ltk.ERR_INVALID),
    ((FAKE, 100, FAKE * 8, 2, 0, FAKE * 64, 0), ltk.ERR_INVALID),    # k = 0
    ((FAKE, 100, FAKE * 8, 2, 129, FAKE * 64, 0), ltk.ERR_UNSUPPORTED),
    ((FAKE, 100, 0, 2, 5, FAKE * 64, 0), ltk.ERR_INVALID),           # NULL offsets
    ((FAKE, 100, FAKE * 8 + 4, 2, 5, FAKE * 64, 0), ltk.ERR_INVALID),  # 4-aligned
    ((FAKE, 100, FAKE * 8, 2, 5, 0, 0), ltk.ERR_INVALID),            # NULL out
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE * 64 + 2, 0), ltk.ERR_INVALID),
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE * 64, FAKE * 32 + 1), ltk.ERR_INVALID),
    ((0, 100, FAKE * 8, 2, 5, FAKE * 64, 0), ltk.ERR_INVALID),       # NULL in
    ((FAKE + 2, 100, FAKE * 8, 2, 5, FAKE * 64, 0), ltk.ERR_INVALID),
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE + 40, 0), ltk.ERR_INVALID),    # out in in
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE * 8 + 8, 0), ltk.ERR_INVALID),  # out on offsets
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE * 64, FAKE * 64 + 20), ltk.ERR_INVALID),
    ((FAKE, 100, FAKE * 8, 2, 5, FAKE * 64, FAKE + 8), ltk.ERR_INVALID),
])
def test_topk_segmented_rejects_invalid_arguments(args, status):
    assert ltk.topk_segmented_raw(*args) == status


def test_topk_segmented_no_segments_is_a_no_op():
    assert ltk.topk_segmented_raw(0, 0, 0, 0, 5, 0) == ltk.OK
    assert ltk.topk_segmented_raw(FAKE, 100, 0, 0, 129, 0) == \
        ltk.ERR_UNSUPPORTED


@pytest.mark.skipif(not no_gpu(), reason="a GPU is visible")
def test_valid_call_without_device_reports_hip_error():
    assert ltk.topk_raw(FAKE, 1000, 20, FAKE * 4) == ltk.ERR_HIP
    assert ltk.topk_noalloc_raw(FAKE, 1000, 20, FAKE * 4) == ltk.ERR_HIP
    assert ltk.reduce_raw(FAKE, 1000, 0, FAKE * 4) == ltk.ERR_HIP
    assert ltk.reduce_raw(0, 0, 1, FAKE * 4) == ltk.ERR_HIP
    assert ltk.stats_raw(FAKE, 1000, FAKE * 4) == ltk.ERR_HIP
    assert ltk.stats_raw(0, 0, FAKE * 4) == ltk.ERR_HIP
    assert ltk.topk_kv_raw(FAKE, 1000, 20, FAKE * 4, FAKE * 8) == ltk.ERR_HIP
    assert ltk.topk_kv_raw(FAKE, 1000, 20, FAKE * 4, FAKE * 8,
                           f32=True) == ltk.ERR_HIP
    assert ltk.topk_batched_raw(FAKE, 4, 100, 100, 5, FAKE * 64) == \
        ltk.ERR_HIP
    assert ltk.topk_merge_raw(FAKE, 8, 20, 20, FAKE * 64) == ltk.ERR_HIP
    assert ltk.histogram_raw(FAKE, 100, 0, 0, 16, FAKE * 64) == ltk.ERR_HIP
    assert ltk.histogram_raw(0, 0, 0, 0, 16, FAKE * 64) == ltk.ERR_HIP
    assert ltk.topk_raw(FAKE, 100000, 5000, FAKE * 64) == ltk.ERR_HIP
    assert ltk.topk_segmented_raw(FAKE, 100, FAKE * 8, 2, 5, FAKE * 64) == \
        ltk.ERR_HIP


def test_grid_setting():
    for bad in (-1, 1025, 1 << 20):
        with pytest.raises(ltk.LibtopkError):
            ltk.set_grid(bad)
    try:
        assert ltk.grid_for(0) == 0
        assert ltk.grid_for(1) == 1
        assert ltk.grid_for(4096 * 3 + 5) == 3   # three full tiles
        ltk.set_grid(7)
        assert ltk.grid_for(10 ** 8) == 7
        assert ltk.grid_for(4096 * 3) == 3       # never more than the tiles
        ltk.set_grid(1024)
        assert ltk.grid_for(10 ** 9) == 1024
    finally:
        ltk.set_grid(0)
    g = ltk.grid_for(10 ** 8)
    assert 1 <= g <= 1024
