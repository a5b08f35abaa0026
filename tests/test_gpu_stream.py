"""The streaming-ceiling helper that bench.py times (tests/hip/focus_stream.hip):
it writes every output vector exactly once with the read vector that maps to
it.  Runs on an MI355X only (marker gpu)."""
import ctypes as ct
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libfocus_stream.so")


@pytest.mark.parametrize("nr,nw", [(1, 1), (1000, 700), (4096, 4096), (100003, 95000), (5000, 0)])
def test_stream_copies_every_output_once(nr, nw):
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libfocus_stream.so is not built (run __graft_entry__.build())")
    lib = ct.CDLL(LIB)
    lib.focus_stream.restype = ct.c_int
    lib.focus_stream.argtypes = [ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_int,
                                 ct.c_int64, ct.c_void_p]
    dev = torch.device("cuda:0")
    src = torch.arange(nr * 4, dtype=torch.int32, device=dev)
    dst = torch.full((max(nw, 1) * 4,), -1, dtype=torch.int32, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    for nt in (0, 1):
        dst.fill_(-1)
        assert lib.focus_stream(src.data_ptr(), nr, dst.data_ptr(), nw, sink.data_ptr(), nt, 0,
                                torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        if nw == 0:
            assert torch.all(dst == -1)
            continue
        j = np.arange(nw, dtype=np.int64)
        first_i = (j * nr + nw - 1) // nw  # smallest i with floor(i * nw / nr) == j
        want = (first_i[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
        assert np.array_equal(dst[: nw * 4].cpu().numpy(), want.astype(np.int32))
