"""The streaming-ceiling helper that bench.py times (tests/hip/focus_stream.hip):
every output it documents, on block counts that leave partial tiles and
partial wavefronts.  Runs on an MI355X only (marker gpu)."""
import ctypes as ct
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libfocus_stream.so")


@pytest.mark.parametrize("u", [1, 2, 4])
@pytest.mark.parametrize("nblk", [1, 63, 64, 513, 100003])
def test_pattern_outputs(nblk, u):
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libfocus_stream.so is not built (run __graft_entry__.build())")
    lib = ct.CDLL(LIB)
    lib.focus_stream_pattern.restype = ct.c_int
    lib.focus_stream_pattern.argtypes = [ct.c_void_p] * 3 + [ct.c_int64] + [ct.c_void_p] * 3 + [ct.c_int, ct.c_void_p]
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(nblk)
    w = torch.randint(-2 ** 31, 2 ** 31 - 1, (nblk * 8,), generator=g, dtype=torch.int64).to(torch.int32)
    m = torch.rand(nblk, generator=g) * 4
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (nblk * 2,), generator=g, dtype=torch.int64).to(torch.int32)
    wd, md, qd = w.to(dev), m.to(dev), q.to(dev)
    codes = torch.zeros(nblk * 2, dtype=torch.int32, device=dev)
    scales = torch.zeros(nblk, dtype=torch.uint8, device=dev)
    wdeq = torch.zeros(nblk * 8, dtype=torch.int32, device=dev)
    assert lib.focus_stream_pattern(wd.data_ptr(), md.data_ptr(), qd.data_ptr(), nblk, codes.data_ptr(),
                                    scales.data_ptr(), wdeq.data_ptr(), u, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    wv = np.concatenate([w.numpy().view(np.uint32).reshape(2 * nblk, 4), np.zeros((128, 4), np.uint32)])
    qn = q.numpy().view(np.uint32).reshape(nblk, 2)
    assert np.array_equal(wdeq.cpu().numpy(), w.numpy())
    b = np.arange(nblk)
    lane, f = b % 64, b // 64
    A, B = wv[128 * f + lane], wv[128 * f + 64 + lane]  # the vectors the block's lane holds
    want = np.stack([A[:, 0] ^ B[:, 1] ^ qn[:, 0], A[:, 2] ^ B[:, 3] ^ qn[:, 1]], 1)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32).reshape(nblk, 2), want)
    assert np.array_equal(scales.cpu().numpy(), ((m.numpy().view(np.uint32) >> 23) & 0xFF).astype(np.uint8))


@pytest.mark.parametrize("tokens,rb,grid", [(1, 4, 1), (9, 1, 2), (8192, 4, 1024), (37, 8, 5)])
def test_act_pattern_outputs(tokens, rb, grid):
    lib = ct.CDLL(LIB)
    lib.focus_stream_act_pattern.restype = ct.c_int
    lib.focus_stream_act_pattern.argtypes = [ct.c_void_p, ct.c_int64, ct.c_int] + [ct.c_void_p] * 3 + [ct.c_int64,
                                                                                                     ct.c_void_p]
    dev = torch.device("cuda:0")
    nb = 64 * rb
    g = torch.Generator(device="cpu").manual_seed(tokens + rb)
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (tokens * nb * 8,), generator=g, dtype=torch.int64).to(torch.int32)
    codes = torch.zeros(tokens * nb * 2, dtype=torch.int32, device=dev)
    scales = torch.zeros(tokens * nb, dtype=torch.uint8, device=dev)
    s2 = torch.zeros(tokens, dtype=torch.float32, device=dev)
    assert lib.focus_stream_act_pattern(x.to(dev).data_ptr(), tokens, rb, codes.data_ptr(), scales.data_ptr(),
                                        s2.data_ptr(), grid, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    xv = x.numpy().view(np.uint32).reshape(tokens, 2 * nb, 4)
    b = np.arange(nb)
    A, B = xv[:, 128 * (b // 64) + b % 64], xv[:, 128 * (b // 64) + 64 + b % 64]
    want = np.stack([A[..., 0] ^ B[..., 1], A[..., 2] ^ B[..., 3]], -1)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32).reshape(tokens, nb, 2), want)
    assert np.array_equal(scales.cpu().numpy().reshape(tokens, nb), ((A[..., 0] ^ B[..., 2]) & 0xFF).astype(np.uint8))
    acc = np.bitwise_xor.reduce(want[:, :, 0].reshape(tokens, rb, 64)[:, :, 0], axis=1) & 0x3FFFFFFF
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), acc.astype(np.uint32))


@pytest.mark.parametrize("u", [4, 8])
@pytest.mark.parametrize("nvec,grid", [(1, 1), (1000, 3), (257 * 8 + 5, 2), (100003, 7)])
def test_read_pattern_outputs(nvec, grid, u):
    lib = ct.CDLL(LIB)
    lib.focus_stream_read_pattern.restype = ct.c_int
    lib.focus_stream_read_pattern.argtypes = [ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_int, ct.c_int64, ct.c_void_p]
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(nvec + u)
    w = torch.randint(-2 ** 31, 2 ** 31 - 1, (nvec * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    out = torch.full((grid * 256,), -1, dtype=torch.int32, device=dev)
    assert lib.focus_stream_read_pattern(w.to(dev).data_ptr(), nvec, out.data_ptr(), u, grid,
                                         torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    wv = w.numpy().view(np.uint32).reshape(nvec, 4)
    x = wv[:, 0] ^ wv[:, 1] ^ wv[:, 2] ^ wv[:, 3]
    i = np.arange(nvec)
    slot = ((i // (256 * u)) % grid) * 256 + i % 256  # the lane that reads vector i
    want = np.zeros(grid * 256, np.uint32)
    np.maximum.at(want, slot, x)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("nblk", [1, 63, 64, 513, 100003])
def test_deq_pattern_outputs(nblk):
    lib = ct.CDLL(LIB)
    lib.focus_stream_deq_pattern.restype = ct.c_int
    lib.focus_stream_deq_pattern.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_void_p]
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(nblk)
    c = torch.randint(-2 ** 31, 2 ** 31 - 1, (nblk * 2,), generator=g, dtype=torch.int64).to(torch.int32)
    s = torch.randint(0, 256, (nblk,), generator=g, dtype=torch.int64).to(torch.uint8)
    out = torch.zeros(nblk * 8 + 8, dtype=torch.int32, device=dev)
    assert lib.focus_stream_deq_pattern(c.to(dev).data_ptr(), s.to(dev).data_ptr(), nblk, out.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    cv = c.numpy().view(np.uint32).reshape(nblk, 2)
    sv = s.numpy().astype(np.uint32)
    want = np.stack([cv[:, 0], cv[:, 1], sv, cv[:, 0] ^ sv, cv[:, 1], cv[:, 0], sv ^ 255, cv[:, 1] ^ sv], 1)
    o = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(o[:nblk * 8].reshape(nblk, 8), want)
    assert not o[nblk * 8:].any()  # nothing written past the end
