"""topk_i32_noalloc, the allocation-free variant of topk_i32: called through
the C ABI on raw device pointers, its output must equal topk_i32's (and the
oracle's), bit for bit, on consecutive calls that share its fixed scratch
array, the second with a smaller input."""
import numpy as np
import pytest

import oracle
import synth
import top_selection_two_amd as ltk

pytestmark = pytest.mark.gpu


def _both(xd, n, k):
    import torch
    ref = torch.empty(k, dtype=torch.int32, device=xd.device)
    got = torch.full((k,), 7, dtype=torch.int32, device=xd.device)
    stream = torch.cuda.current_stream(xd.device).cuda_stream
    assert ltk.topk_raw(xd.data_ptr(), n, k, ref.data_ptr(), stream) == ltk.OK
    assert ltk.topk_noalloc_raw(xd.data_ptr(), n, k, got.data_ptr(),
                                stream) == ltk.OK
    return got.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("sizes", [
    ((3_000_017, 20), (100_003, 20)),     # many workgroups, then fewer
    ((10_000_000, 128), (1_000_001, 7)),  # largest list, then the smallest
    ((5_000, 100), (301, 1)),             # one tile and less
])
def test_noalloc_matches_topk_on_two_calls(sizes):
    import torch
    dev = torch.device("cuda:0")
    for n, k in sizes:
        x = synth.workload("full_1e6", n=n)
        xd = torch.from_numpy(x).to(dev)
        got, ref = _both(xd, n, k)
        print("noalloc n=%d k=%d" % (n, k), flush=True)
        assert np.array_equal(got, ref)
        assert np.array_equal(got, oracle.topk(x, k))


def test_noalloc_heavy_ties_then_small():
    import torch
    dev = torch.device("cuda:0")
    x = synth.workload("dup1000_1e7", n=2_000_000)
    xd = torch.from_numpy(x).to(dev)
    got, ref = _both(xd, x.size, 100)
    assert np.array_equal(got, ref)
    assert np.array_equal(got, oracle.topk(x, 100))
    y = np.sort(x[:40_000])
    yd = torch.from_numpy(y).to(dev)
    got, ref = _both(yd, y.size, 64)
    assert np.array_equal(got, ref)
    assert np.array_equal(got, oracle.topk(y, 64))


def test_noalloc_rejects_large_k():
    import torch
    dev = torch.device("cuda:0")
    xd = torch.zeros(1000, dtype=torch.int32, device=dev)
    out = torch.empty(200, dtype=torch.int32, device=dev)
    assert ltk.topk_noalloc_raw(xd.data_ptr(), 1000, 129,
                                out.data_ptr()) == ltk.ERR_UNSUPPORTED
    assert ltk.topk_noalloc_raw(xd.data_ptr(), 1000, 0,
                                out.data_ptr()) == ltk.ERR_INVALID
