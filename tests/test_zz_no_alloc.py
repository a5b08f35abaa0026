"""focus_nvfp4_linear_noalloc (the linear layer with the library's per-GPU
scratch as its split-k workspace, for callers that cannot allocate) against
focus_nvfp4_linear given a caller workspace of the same size, through the C
ABI: bit-identical outputs, on two calls in a row whose second input is
smaller (the scratch keeps the first call's partials), for shapes that split
k on the decode kernel and on the tiled kernel, one of them a split that
fills the whole scratch.  MI355X only (marker gpu)."""
import ctypes as ct

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def lib():
    import fp4_post_weight_amd as f
    return f._lib.lib()


def _operands(M, N, K, seed):
    xc, xs = synth.nvfp4_operand(M, K, seed=seed, tensor_id=50, device=DEV)
    wc, ws = synth.nvfp4_operand(N, K, seed=seed, tensor_id=51, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(seed)
    s2x = (torch.rand(M, generator=g) * 1e-2 + 1e-3).to(DEV)
    s2w = torch.tensor([3e-3], dtype=torch.float32, device=DEV)
    return xc, xs, s2x, wc, ws, s2w


def _reference(lib, ops, M, N, K, y_dtype, ws_bytes):
    xc, xs, s2x, wc, wsc, s2w = ops
    y = torch.empty((M, N), dtype=torch.float32 if y_dtype == 0 else torch.bfloat16, device=DEV)
    wsp = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=DEV)
    st = lib.focus_nvfp4_linear(xc.data_ptr(), xs.data_ptr(), s2x.data_ptr(), 1, M, wc.data_ptr(), wsc.data_ptr(),
                                s2w.data_ptr(), N, K, y.data_ptr(), y_dtype, wsp.data_ptr() if ws_bytes else None,
                                ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    return y


def _noalloc(lib, ops, M, N, K, y_dtype):
    xc, xs, s2x, wc, wsc, s2w = ops
    y = torch.full((M, N), float("nan"), dtype=torch.float32 if y_dtype == 0 else torch.bfloat16, device=DEV)
    st = lib.focus_nvfp4_linear_noalloc(xc.data_ptr(), xs.data_ptr(), s2x.data_ptr(), 1, M, wc.data_ptr(),
                                        wsc.data_ptr(), s2w.data_ptr(), N, K, y.data_ptr(), y_dtype,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    return y


# (first call, second smaller call): decode kernel with a k split, tiled
# kernel with a k split, and a tiled split of 256 workgroups of 256 x 256
# outputs, whose FP32 partials take the whole 64 MiB
PAIRS = [((16, 1024, 28672), (8, 512, 14336)),
         ((512, 4096, 4096), (300, 2048, 2048)),
         ((1024, 1024, 28672), (1024, 1024, 4096))]


@pytest.mark.parametrize("y_dtype", [0, 1], ids=["f32", "bf16"])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}x{p[0][1]}x{p[0][2]}")
def test_noalloc_matches_workspace_call(lib, pair, y_dtype):
    cap = int(lib.focus_nvfp4_linear_scratch_bytes())
    assert cap == 64 << 20
    for n, (M, N, K) in enumerate(pair):
        ws_full = int(lib.focus_nvfp4_linear_workspace_bytes(M, N, K))
        assert ws_full >= 0
        print(f"call {n}: M={M} N={N} K={K} full split workspace {ws_full} B, scratch {cap} B", flush=True)
        ops = _operands(M, N, K, seed=7 + n)
        ref = _reference(lib, ops, M, N, K, y_dtype, min(ws_full, cap))
        got = _noalloc(lib, ops, M, N, K, y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), (M, N, K)
    # the shapes exercise the split: on this GPU every first call splits k
    assert int(lib.focus_nvfp4_linear_workspace_bytes(*pair[0])) > 0


def test_noalloc_validation_and_binding(lib):
    import fp4_post_weight_amd as f
    FAKE = 0x10000
    g = lib.focus_nvfp4_linear_noalloc
    assert g(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 60, FAKE, 0, None) == 2   # K % 16
    assert g(FAKE, FAKE, FAKE, 2, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == 5   # per-row flag
    assert g(FAKE, FAKE, None, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == 1   # NULL s2
    assert g(FAKE + 4, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == 3
    assert g(None, None, None, 1, 0, None, None, None, 8, 64, None, 0, None) == 0   # empty
    # the binding: same result as nvfp4_linear, and an undersized out is refused
    M, N, K = 16, 1024, 28672
    xc, xs, s2x, wc, wsc, s2w = _operands(M, N, K, seed=3)
    x = f.Quantized(xc, xs, None, s2x)
    w = f.Quantized(wc, wsc, None, s2w)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    f.nvfp4_linear_noalloc(x, w, out)
    ref = f.nvfp4_linear(x, w, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    with pytest.raises(ValueError):
        f.nvfp4_linear_noalloc(x, w, out[:8])
