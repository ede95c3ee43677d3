"""Python binding for libtopk (two-stage reduction and Top-K on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libtopk.so, whose C interface is include/libtopk.h.  PyTorch
supplies device memory and the current stream.  There is no CPU fallback:
if the library is not built, importing this package raises.

    topk(x, k)      -> int32 tensor [k], the k largest of x, descending
    reduce(x, op)   -> int64 tensor [1]: SUM, MAX or MIN of x
    topk_kv(x, k)   -> (values [k], int64 positions [k]) of an int32 or
                       float32 x: value descending, then position ascending
    stats(x)        -> int64 tensor [6]: count, sum, max, min and the sum of
                       squares (low, high 64 bits) of x, from one read
    unpack_stats(t) -> the same as a dict of Python ints (sum of squares
                       joined into one integer)
    topk_batched(x, k, cols=None)
                    -> int32 tensor [rows, k]: the top-k of every row of the
                       2-D int32 x (rows may be strided; with cols, only the
                       first cols columns of each row count)
    topk_merge(lists, k)
                    -> int32 tensor [k]: the k largest of the union of the
                       rows of lists (each row in descending order)
    histogram(x, lo, shift, nbins)
                    -> int64 tensor [nbins]: counts of x in bins of width
                       2**shift starting at lo
    topk_segmented(x, offsets, k)
                    -> (int32 [nseg, k], int32 counts [nseg]): the top-k of
                       every segment x[offsets[s] .. offsets[s+1])
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libtopk.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_NOMEM, ERR_HIP = 0, 1, 2, 3, 4
MAX_K_SELECT = 16384   # LIBTOPK_MAX_K_SELECT: largest k of topk()
MAX_BINS = 4096        # LIBTOPK_MAX_BINS
SUM, MAX, MIN = 0, 1, 2
OPS = {"sum": SUM, "max": MAX, "min": MIN}

# Entry points of include/libtopk.h with their ctypes signatures.
_VP = ctypes.c_void_p
SIGNATURES = {
    "topk_i32": ([_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP],
                 ctypes.c_int),
    "topk_i32_noalloc": ([_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP],
                         ctypes.c_int),
    "reduce_i32": ([_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP],
                   ctypes.c_int),
    "reduce_stats_i32": ([_VP, ctypes.c_int64, _VP, _VP], ctypes.c_int),
    "topk_kv_i32": ([_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP, _VP],
                    ctypes.c_int),
    "topk_kv_f32": ([_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP, _VP],
                    ctypes.c_int),
    "topk_batched_i32": ([_VP, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_int64, ctypes.c_int32, _VP, _VP],
                         ctypes.c_int),
    "topk_merge_i32": ([_VP, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                        _VP, _VP], ctypes.c_int),
    "topk_segmented_i32": ([_VP, ctypes.c_int64, _VP, ctypes.c_int64,
                            ctypes.c_int32, _VP, _VP, _VP], ctypes.c_int),
    "histogram_i32": ([_VP, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, _VP, _VP], ctypes.c_int),
    "libtopk_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "libtopk_max_k": ([], ctypes.c_int),
    "libtopk_set_grid": ([ctypes.c_int32], ctypes.c_int),
    "libtopk_grid_for": ([ctypes.c_int64], ctypes.c_int32),
    "libtopk_debug_scramble": ([_VP, ctypes.c_int32, ctypes.c_uint64],
                               ctypes.c_int),
    "libtopk_release": ([], None),
}


class LibtopkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)"
                         % (what, strerror(status), status))


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime.  Tensors and streams handed to the
    # library come from that runtime, so it must be the one libtopk.so binds
    # to: loading torch first makes its libamdhip64 satisfy the library's
    # dependency (same soname) instead of a second runtime from /opt/rocm.
    import torch  # noqa: F401
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            "libtopk.so is not built (expected at %s); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` from the "
            "repository root" % LIBRARY_PATH)
    lib = ctypes.CDLL(LIBRARY_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.libtopk_strerror(status).decode()


def max_k() -> int:
    return lib.libtopk_max_k()


def set_grid(blocks: int) -> None:
    """Stage-1 workgroups for later calls (0 = automatic)."""
    rc = lib.libtopk_set_grid(blocks)
    if rc != OK:
        raise LibtopkError(rc, "libtopk_set_grid")


def grid_for(n: int) -> int:
    return int(lib.libtopk_grid_for(n))


def release() -> None:
    lib.libtopk_release()


def debug_scramble(which: int = 0, seed: int = 1, stream: int | None = None):
    """Overwrite the tickets and histogram counters that later calls on the
    current stream (which=0) or topk_i32_noalloc (which=1) use with
    pseudo-random words: no result may depend on them (a test hook)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib.libtopk_debug_scramble(stream or None, which,
                                    seed & (2 ** 64 - 1))
    if rc != OK:
        raise LibtopkError(rc, "libtopk_debug_scramble")


# ---------------------------------------------------------------- raw calls
def topk_raw(in_ptr: int, n: int, k: int, out_ptr: int, stream: int = 0) -> int:
    """Call topk_i32 on raw device pointers; returns the status code."""
    return lib.topk_i32(in_ptr or None, n, k, out_ptr or None, stream or None)


def topk_noalloc_raw(in_ptr: int, n: int, k: int, out_ptr: int,
                     stream: int = 0) -> int:
    """Call topk_i32_noalloc on raw device pointers; returns the status."""
    return lib.topk_i32_noalloc(in_ptr or None, n, k, out_ptr or None,
                                stream or None)


def reduce_raw(in_ptr: int, n: int, op: int, out_ptr: int,
               stream: int = 0) -> int:
    """Call reduce_i32 on raw device pointers; returns the status code."""
    return lib.reduce_i32(in_ptr or None, n, op, out_ptr or None,
                          stream or None)


def stats_raw(in_ptr: int, n: int, out_ptr: int, stream: int = 0) -> int:
    """Call reduce_stats_i32 on raw device pointers; returns the status."""
    return lib.reduce_stats_i32(in_ptr or None, n, out_ptr or None,
                                stream or None)


def topk_kv_raw(in_ptr: int, n: int, k: int, vals_ptr: int, idx_ptr: int,
                stream: int = 0, f32: bool = False) -> int:
    """Call topk_kv_i32 (or topk_kv_f32) on raw device pointers."""
    fn = lib.topk_kv_f32 if f32 else lib.topk_kv_i32
    return fn(in_ptr or None, n, k, vals_ptr or None, idx_ptr or None,
              stream or None)


def topk_batched_raw(in_ptr: int, rows: int, cols: int, ld: int, k: int,
                     out_ptr: int, stream: int = 0) -> int:
    """Call topk_batched_i32 on raw device pointers; returns the status."""
    return lib.topk_batched_i32(in_ptr or None, rows, cols, ld, k,
                                out_ptr or None, stream or None)


def topk_merge_raw(lists_ptr: int, m: int, length: int, k: int, out_ptr: int,
                   stream: int = 0) -> int:
    """Call topk_merge_i32 on raw device pointers; returns the status."""
    return lib.topk_merge_i32(lists_ptr or None, m, length, k,
                              out_ptr or None, stream or None)


def topk_segmented_raw(in_ptr: int, n: int, offsets_ptr: int, nseg: int,
                       k: int, out_ptr: int, counts_ptr: int = 0,
                       stream: int = 0) -> int:
    """Call topk_segmented_i32 on raw device pointers; returns the status."""
    return lib.topk_segmented_i32(in_ptr or None, n, offsets_ptr or None,
                                  nseg, k, out_ptr or None, counts_ptr or None,
                                  stream or None)


def histogram_raw(in_ptr: int, n: int, lo: int, shift: int, nbins: int,
                  out_ptr: int, stream: int = 0) -> int:
    """Call histogram_i32 on raw device pointers; returns the status."""
    return lib.histogram_i32(in_ptr or None, n, lo, shift, nbins,
                             out_ptr or None, stream or None)


# ---------------------------------------------------------------- tensors
def _check_input(x, dtypes=("int32",)):
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if str(x.dtype).replace("torch.", "") not in dtypes:
        raise TypeError("expected %s, got %s" % (" or ".join(dtypes), x.dtype))
    if x.device.type != "cuda":
        raise ValueError("expected a device tensor, got %s" % x.device)
    if x.dim() != 1 or not x.is_contiguous():
        raise ValueError("expected a contiguous 1-D tensor")


def topk(x, k: int, out=None):
    """The k largest values of the int32 device tensor x, descending."""
    import torch
    _check_input(x)
    if out is None:
        out = torch.empty(max(int(k), 0), dtype=torch.int32, device=x.device)
    elif (out.dtype != torch.int32 or out.device != x.device
          or out.numel() != k or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [k] tensor on "
                         "x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.topk_i32(x.data_ptr() if x.numel() else None, x.numel(), k,
                          out.data_ptr() if out.numel() else None,
                          stream or None)
    if rc != OK:
        raise LibtopkError(rc, "topk_i32")
    return out


def reduce(x, op, out=None):
    """SUM (exact int64), MAX or MIN of the int32 device tensor x."""
    import torch
    _check_input(x)
    if isinstance(op, str):
        op = OPS[op]
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=x.device)
    elif (out.dtype != torch.int64 or out.device != x.device
          or out.numel() != 1):
        raise ValueError("out must be an int64 [1] tensor on x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.reduce_i32(x.data_ptr() if x.numel() else None, x.numel(),
                            op, out.data_ptr(), stream or None)
    if rc != OK:
        raise LibtopkError(rc, "reduce_i32")
    return out


def stats(x, out=None):
    """count, sum, max, min, sum of squares (low, high) of the int32 device
    tensor x, as an int64 device tensor [6] (see reduce_stats_i32)."""
    import torch
    _check_input(x)
    if out is None:
        out = torch.empty(6, dtype=torch.int64, device=x.device)
    elif (out.dtype != torch.int64 or out.device != x.device
          or out.numel() != 6 or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int64 [6] tensor on x's "
                         "device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.reduce_stats_i32(x.data_ptr() if x.numel() else None,
                                  x.numel(), out.data_ptr(), stream or None)
    if rc != OK:
        raise LibtopkError(rc, "reduce_stats_i32")
    return out


def unpack_stats(t) -> dict:
    """The [6] result of stats() as Python ints (copies to the host)."""
    v = [int(a) for a in t.cpu().tolist()]
    lo, hi = v[4] & (2 ** 64 - 1), v[5] & (2 ** 64 - 1)
    return {"count": v[0], "sum": v[1], "max": v[2], "min": v[3],
            "sumsq": lo | (hi << 64)}


def topk_kv(x, k: int, out=None):
    """The k largest elements of the int32 or float32 device tensor x and
    their positions: (values [k] of x's dtype, int64 positions [k]), ordered
    by value descending, then position ascending (see topk_kv_i32)."""
    import torch
    _check_input(x, ("int32", "float32"))
    if out is None:
        vals = torch.empty(max(int(k), 0), dtype=x.dtype, device=x.device)
        idx = torch.empty(max(int(k), 0), dtype=torch.int64, device=x.device)
    else:
        vals, idx = out
        if (vals.dtype != x.dtype or idx.dtype != torch.int64
                or vals.numel() != k or idx.numel() != k
                or vals.device != x.device or idx.device != x.device
                or not vals.is_contiguous() or not idx.is_contiguous()):
            raise ValueError("out must be contiguous ([k] of x's dtype, "
                             "int64 [k]) on x's device")
    fn = lib.topk_kv_f32 if x.dtype == torch.float32 else lib.topk_kv_i32
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = fn(x.data_ptr() if x.numel() else None, x.numel(), k,
                vals.data_ptr() if vals.numel() else None,
                idx.data_ptr() if idx.numel() else None, stream or None)
    if rc != OK:
        raise LibtopkError(rc, fn.__name__)
    return vals, idx


def _check_rows(x):
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if x.dtype != torch.int32:
        raise TypeError("expected int32, got %s" % x.dtype)
    if x.device.type != "cuda":
        raise ValueError("expected a device tensor, got %s" % x.device)
    if x.dim() != 2 or x.stride(1) != 1 or (x.size(0) > 1
                                            and x.stride(0) < x.size(1)):
        raise ValueError("expected a 2-D tensor with unit column stride and "
                         "row stride >= its row length")


def topk_batched(x, k: int, cols: int | None = None, out=None):
    """Top-k of every row of the 2-D int32 device tensor x (row stride
    x.stride(0), unit column stride): an int32 tensor [rows, k], each row
    descending.  With cols, only the first cols columns of each row count."""
    import torch
    _check_rows(x)
    rows, width = x.shape
    c = width if cols is None else int(cols)
    if c > width:
        raise ValueError("cols exceeds the tensor's row length")
    ld = x.stride(0) if rows > 1 else max(width, 1)
    if out is None:
        out = torch.empty((rows, max(int(k), 0)), dtype=torch.int32,
                          device=x.device)
    elif (out.dtype != torch.int32 or out.device != x.device
          or out.numel() != rows * k or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [rows, k] tensor on "
                         "x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.topk_batched_i32(x.data_ptr() if x.numel() else None, rows,
                                  c, ld, k,
                                  out.data_ptr() if out.numel() else None,
                                  stream or None)
    if rc != OK:
        raise LibtopkError(rc, "topk_batched_i32")
    return out


def topk_merge(lists, k: int, out=None):
    """The k largest values of the union of the rows of the 2-D int32 device
    tensor `lists` (contiguous; each row in descending order), descending."""
    import torch
    _check_rows(lists)
    if not lists.is_contiguous():
        raise ValueError("expected a contiguous 2-D tensor")
    m, length = lists.shape
    if out is None:
        out = torch.empty(max(int(k), 0), dtype=torch.int32,
                          device=lists.device)
    elif (out.dtype != torch.int32 or out.device != lists.device
          or out.numel() != k or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [k] tensor on the "
                         "lists' device")
    with torch.cuda.device(lists.device):
        stream = torch.cuda.current_stream(lists.device).cuda_stream
        rc = lib.topk_merge_i32(lists.data_ptr() if lists.numel() else None,
                                m, length, k,
                                out.data_ptr() if out.numel() else None,
                                stream or None)
    if rc != OK:
        raise LibtopkError(rc, "topk_merge_i32")
    return out


def topk_segmented(x, offsets, k: int, out=None, counts=None,
                   with_counts: bool = True):
    """Top-k of every segment x[offsets[s] .. offsets[s+1]) of the 1-D int32
    device tensor x; offsets is an int64 device tensor of nseg + 1
    non-decreasing entries within [0, x.numel()].  Returns (out, counts):
    an int32 tensor [nseg, k], each row descending and padded with INT32_MIN
    past a short segment's values, and the int32 counts [nseg] =
    min(k, length) (None when with_counts is False)."""
    import torch
    _check_input(x)
    if (not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int64
            or offsets.device != x.device or offsets.dim() != 1
            or offsets.numel() < 1 or not offsets.is_contiguous()):
        raise ValueError("offsets must be a contiguous 1-D int64 tensor of "
                         "nseg + 1 entries on x's device")
    nseg = offsets.numel() - 1
    if out is None:
        out = torch.empty((nseg, max(int(k), 0)), dtype=torch.int32,
                          device=x.device)
    elif (out.dtype != torch.int32 or out.device != x.device
          or out.numel() != nseg * k or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [nseg, k] tensor on "
                         "x's device")
    if with_counts and counts is None:
        counts = torch.empty(nseg, dtype=torch.int32, device=x.device)
    elif counts is not None and (counts.dtype != torch.int32
                                 or counts.device != x.device
                                 or counts.numel() != nseg
                                 or not counts.is_contiguous()):
        raise ValueError("counts must be a contiguous int32 [nseg] tensor on "
                         "x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.topk_segmented_i32(
            x.data_ptr() if x.numel() else None, x.numel(),
            offsets.data_ptr(), nseg, k,
            out.data_ptr() if out.numel() else None,
            counts.data_ptr() if counts is not None and nseg else None,
            stream or None)
    if rc != OK:
        raise LibtopkError(rc, "topk_segmented_i32")
    return out, counts


def histogram(x, lo: int, shift: int, nbins: int, out=None):
    """int64 counts of the int32 device tensor x in nbins bins of width
    2**shift starting at lo (see histogram_i32)."""
    import torch
    _check_input(x)
    if out is None:
        out = torch.empty(max(int(nbins), 0), dtype=torch.int64,
                          device=x.device)
    elif (out.dtype != torch.int64 or out.device != x.device
          or out.numel() != nbins or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int64 [nbins] tensor on "
                         "x's device")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.histogram_i32(x.data_ptr() if x.numel() else None,
                               x.numel(), lo, shift, nbins,
                               out.data_ptr() if out.numel() else None,
                               stream or None)
    if rc != OK:
        raise LibtopkError(rc, "histogram_i32")
    return out
