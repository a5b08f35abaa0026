"""The NVFP4 linear layer Y = X' W'^T on the matrix cores (through the C
ABI) against the oracle's binary64 definition.  MI355X only (marker gpu).

Bound (derived from the arithmetic): every c*S is exact in FP16 and every
product exact in FP32; the FP32 accumulation of K products in any order errs
by at most (K - 1) roundings of at most 2^-23 relative each (round-to-nearest
gives 2^-24; 2^-23 also covers truncation), and two more roundings come from
s2x*s2w and the final product, so
    |Y - exact| <= (2K + 4) * 2^-24 * sum_k |products| * s2x * s2w,
plus half a BF16 spacing (2^-9 |Y|, 2^-8 taken) for BF16 output.  When all
scales are 1 and the s2 are powers of two every partial sum is exact in FP32
and Y must equal the oracle bit for bit; that case pins the operand and
output layouts exactly.  Inputs are random NVFP4 bytes (synth.nvfp4_operand),
never outputs of the HIP path.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import parity
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def focus():
    import fp4_post_weight_amd as f
    f._lib.lib()
    assert torch.cuda.is_available()
    return f


def operands(M, N, K, seed, **kw):
    xc, xs = synth.nvfp4_operand(M, K, seed=seed, tensor_id=40, **kw)
    wc, ws = synth.nvfp4_operand(N, K, seed=seed, tensor_id=41, **kw)
    return xc, xs, wc, ws


def oracle_linear(orc, xc, xs, s2x, wc, ws, s2w):
    """The oracle over row chunks of X on all host threads."""
    M = xc.shape[0]
    n = max(1, min(parity.threads(), M))
    bounds = np.linspace(0, M, n + 1).astype(int)
    s2x = np.atleast_1d(s2x)

    def run(i):
        a, b = bounds[i], bounds[i + 1]
        return orc.nvfp4_linear(xc[a:b], xs[a:b], s2x[a:b] if s2x.size == M else s2x, wc, ws, s2w)

    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(run, range(n)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, out_dtype, workspace="auto"):
    x = focus.Quantized(xc.to(DEV), xs.to(DEV), None, torch.as_tensor(s2x, dtype=torch.float32).reshape(-1).to(DEV))
    w = focus.Quantized(wc.to(DEV), ws.to(DEV), None, torch.tensor([s2w], dtype=torch.float32, device=DEV))
    y = focus.nvfp4_linear(x, w, out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def check_bound(y, ref, refabs, K, bf16, label):
    bound = (2 * K + 4) * 2.0 ** -24 * refabs
    if bf16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(y - ref)
    bad = err > bound
    assert not bad.any(), (f"{label}: {bad.sum()} outputs outside the bound; worst at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)}")
    return float(np.max(err / np.maximum(refabs, 1e-300)))


@pytest.mark.parametrize("M", [300, 100, 40, 32, 16, 5], ids=lambda v: f"M{v}")
def test_exact_when_partial_sums_are_exact(focus, orc, M):
    # M = 300: tiled kernel; 100: decode kernel with eight 16-token X tiles,
    # 40 with four, 32 with two, 16 and 5 with one (operand and output
    # layouts of each)
    N, K = 520, 1024
    xc, _, wc, _ = operands(M, N, K, 1)
    xs = torch.full((M, K // 16), 0x38, dtype=torch.uint8)
    ws = torch.full((N, K // 16), 0x38, dtype=torch.uint8)
    s2x = np.exp2(-(np.arange(M) % 7)).astype(np.float32)
    s2w = np.float32(0.125)
    ref, _ = oracle_linear(orc, xc.numpy(), xs.numpy(), s2x, wc.numpy(), ws.numpy(), s2w)
    y32 = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, torch.float32)
    assert np.array_equal(y32, ref), f"{np.count_nonzero(y32 != ref)} FP32 outputs differ"
    y16 = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, torch.bfloat16)
    want = torch.from_numpy(ref).float().to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(y16, want)


# M <= 128 takes the decode kernel (1, 2, 4 or 8 tiles of 16 tokens; K % 256
# != 0: masked loads; K % 256 == 0 with up to 4 token tiles and 2 column tiles
# per wavefront: W through the wavefront's LDS area), larger M the tiled
# kernel (K % 64 != 0: masked loads); some shapes split k.
SHAPES = [(1, 1, 16), (3, 17, 256), (7, 33, 48), (12, 4111, 320), (16, 200, 1040), (16, 4096, 4096),
          (5, 1000, 28672), (16, 1024, 28688), (1, 14336, 512), (3, 8200, 80), (20, 8192, 256), (50, 8200, 512),
          (17, 64, 64), (32, 4096, 4096), (33, 1000, 1040), (64, 512, 8192), (64, 300, 14336),
          (32, 1000, 28672), (100, 520, 28672), (100, 8200, 80), (65, 130, 192), (100, 8200, 512), (128, 1000, 4160), (129, 130, 192), (255, 257, 64), (257, 255, 1040),
          (300, 520, 4096), (513, 96, 80),
          (16, 16400, 256), (9, 16448, 1040),  # two 16-column tiles per wavefront, through LDS and direct, ragged
          (16, 6200, 512),  # two tiles at three workgroups per four CUs, ragged
          (16, 4100, 8224),  # 16 wavefronts per workgroup (33 k-steps, the last one masked), ragged
          (24, 16400, 512),  # two tiles with 2 token tiles
          (16, 24600, 256), (24, 24600, 512),  # two tiles, 4 wavefronts at three workgroups per CU, ragged
          (33, 16448, 2064), (33, 16400, 1024), (100, 16400, 256),  # four tiles with 4 and 8 token tiles
          (33, 6200, 512), (97, 6200, 1040),  # two tiles at three workgroups per four CUs, 4 and 8 token tiles
          (7, 1000, 4096),  # one tile through LDS, rows past N read the last row, ragged
          (5, 8180, 8192)]  # 16 wavefronts with two tiles (32 k-steps, a workgroup per CU), ragged


@pytest.mark.parametrize("M,N,K", SHAPES, ids=lambda v: str(v))
def test_linear_within_bound(focus, orc, M, N, K):
    """Every shape with the split-k workspace (split wherever the output has
    few tiles) and without it; the split result is also run-to-run
    identical."""
    xc, xs, wc, ws = operands(M, N, K, M + N + K)
    rng = np.random.default_rng(K)
    s2x = (rng.uniform(0.5, 2.0, M) * 2.0 ** -9).astype(np.float32)
    s2w = np.float32(3.0e-4)
    ref, refabs = oracle_linear(orc, xc.numpy(), xs.numpy(), s2x, wc.numpy(), ws.numpy(), s2w)
    for dt in (torch.float32, torch.bfloat16):
        y = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, dt)
        check_bound(y, ref, refabs, K, dt == torch.bfloat16, f"{(M, N, K)} {dt}")
        y2 = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, dt)
        assert np.array_equal(y, y2), "split-k result differs between runs"
        y0 = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, dt, workspace=None)
        check_bound(y0, ref, refabs, K, dt == torch.bfloat16, f"{(M, N, K)} {dt} no workspace")


def _random_shapes(n, seed):
    """Seeded random shapes over the decode and tiled kernels' configurations:
    M in each token-tile band and past 128, N from one column to a few
    thousand (ragged tiles), K aligned to 256 (LDS-staged loads in the decode
    kernel) or not (masked loads), M * N * K kept small for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 7, 16, 17, 31, 32, 33, 48, 64, 65, 100, 128, 129, 200]))
        N = int(rng.integers(1, 4000))
        K = int(256 * rng.integers(1, 24) + (0 if i % 2 == 0 else 16 * rng.integers(1, 16)))
        while M * N * K > 60_000_000:
            N = max(1, N // 2)
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(40, 2026), ids=lambda v: str(v))
def test_linear_random_shapes(focus, orc, M, N, K):
    """Seeded random shapes within the derived bound, with and without the
    split-k workspace."""
    xc, xs, wc, ws = operands(M, N, K, 7 * M + 3 * N + K)
    rng = np.random.default_rng(N)
    s2x = (rng.uniform(0.5, 2.0, M) * 2.0 ** -9).astype(np.float32)
    s2w = np.float32(2.5e-4)
    ref, refabs = oracle_linear(orc, xc.numpy(), xs.numpy(), s2x, wc.numpy(), ws.numpy(), s2w)
    for ws_arg in ("auto", None):
        y = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, torch.bfloat16, workspace=ws_arg)
        check_bound(y, ref, refabs, K, True, f"{(M, N, K)} workspace={ws_arg}")


@pytest.mark.parametrize("M,N,K", [(16, 1024, 28672), (100, 520, 28672), (8, 14336, 512), (2048, 1024, 4096)],
                         ids=lambda v: str(v))
def test_linear_deterministic(focus, M, N, K):
    """Repeated calls give bit-identical outputs on every path, the split ones
    included (partials are summed in range order, workgroup partial tiles in
    wavefront order; no atomics)."""
    xc, xs, wc, ws = operands(M, N, K, 17)
    s2x = np.full(M, 1e-3, dtype=np.float32)
    assert focus.nvfp4_linear_workspace_bytes(M, N, K) > 0 or N == 14336  # the split paths split
    ys = [gpu_linear(focus, xc, xs, s2x, wc, ws, np.float32(1e-3), torch.float32) for _ in range(3)]
    assert all(np.array_equal(ys[0].view(np.uint64), y.view(np.uint64)) for y in ys[1:])


@pytest.mark.parametrize("M", [130, 9, 100], ids=lambda v: f"M{v}")
def test_linear_single_activation_scale_and_wide_scales(focus, orc, M):
    N, K = 200, 512
    xc, xs, wc, ws = operands(M, N, K, 5, scale_lo=0x01, scale_hi=0x7F)  # subnormal to 448
    ref, refabs = oracle_linear(orc, xc.numpy(), xs.numpy(), np.float32(0.02), wc.numpy(), ws.numpy(),
                                np.float32(0.001))
    y = gpu_linear(focus, xc, xs, np.float32(0.02), wc, ws, np.float32(0.001), torch.float32)
    check_bound(y, ref, refabs, K, False, "one s2x, scale bytes 0x01..0x7E")


@pytest.mark.parametrize("M,N,K", [(16, 200, 1024), (130, 300, 512), (140, 90, 1040)], ids=lambda v: str(v))
def test_linear_signed_and_nan_scales(focus, orc, M, N, K):
    """Scale bytes with either sign over 0x00..0x7E (zero, subnormal, normal)
    and the NaN bytes 0x7F / 0xFF planted in a few rows of X and W: an output
    is NaN exactly where the oracle's is (a NaN block scale poisons its row
    even against zero codes), and every other output is within the bound.
    The three shapes take the decode, tiled and masked-load paths."""
    xc, xs, wc, ws = operands(M, N, K, 11, scale_lo=0x00, scale_hi=0x7F)
    g = torch.Generator().manual_seed(M * N + K)
    xs = xs | (torch.randint(0, 2, xs.shape, generator=g, dtype=torch.uint8) << 7)
    ws = ws | (torch.randint(0, 2, ws.shape, generator=g, dtype=torch.uint8) << 7)
    for t, b, v in ((0, 0, 0x7F), (M - 1, K // 16 - 1, 0xFF), (M // 2, 1, 0x7F)):
        xs[t, b] = v
    for o, b, v in ((1, K // 16 - 1, 0xFF), (N - 2, 0, 0x7F)):
        ws[o, b] = v
    s2x, s2w = np.float32(0.01), np.float32(0.002)
    ref, refabs = oracle_linear(orc, xc.numpy(), xs.numpy(), s2x, wc.numpy(), ws.numpy(), s2w)
    nan = np.isnan(ref)
    assert nan.any() and not nan.all()
    for dt in (torch.float32, torch.bfloat16):
        y = gpu_linear(focus, xc, xs, s2x, wc, ws, s2w, dt)
        assert np.array_equal(np.isnan(y), nan), f"{dt}: NaN pattern differs"
        check_bound(np.where(nan, 0.0, y), np.where(nan, 0.0, ref), np.where(nan, 0.0, refabs), K,
                    dt == torch.bfloat16, f"{(M, N, K)} {dt} signed scales")


@pytest.mark.parametrize("M", [1, 33, 129])
@pytest.mark.parametrize("nb", [256, 254])
@pytest.mark.parametrize("side", ["x", "w"])
def test_linear_every_scale_byte(focus, side, nb, M):
    """Closed form over every E4M3 scale byte except NaN: one operand's block
    scales run through all byte values (signed zeros, subnormals, normals up
    to +-448) and the other operand is one-hot, so each output is exactly
    one scale's value, Y[t, o] = E4M3(byte of output o), in FP32 and in BF16
    (at most 4 significant bits; the -0 byte reads as +0 because the FP32
    sum starts from +0).  Expected values come from torch's
    float8_e4m3fn decoding.  nb = 256 blocks (K % 64 == 0, the 0x7F / 0xFF
    slots refilled with 0x38) takes the aligned loads, 254 the masked ones;
    M = 1 and 33 the decode kernel (one and four token tiles), 129 the tiled
    one."""
    byts = [b for b in range(256) if (b & 0x7F) != 0x7F]
    if nb == 256:
        byts = [b if (b & 0x7F) != 0x7F else 0x38 for b in range(256)]
    K, N = 16 * nb, nb
    sel = torch.tensor(byts, dtype=torch.uint8)
    want = sel.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    one = np.uint8(0x02)  # E2M1 1.0 in the low nibble: element 16 j of byte 8 j
    if side == "x":
        # X row: block j has scale byts[j] and a 1.0 at element 16 j; W row o
        # is 1.0 at element 16 o under unit scales
        xc = torch.zeros((M, K // 2), dtype=torch.uint8)
        xc[:, 8 * torch.arange(nb)] = one
        xs = sel.repeat(M, 1)
        wc = torch.zeros((N, K // 2), dtype=torch.uint8)
        wc[torch.arange(N), 8 * torch.arange(N)] = one
        ws = torch.full((N, nb), 0x38, dtype=torch.uint8)
    else:
        # W row o: block 0 has scale byts[o] and a 1.0 at element 0; X row is
        # 1.0 at element 0 under unit scales
        xc = torch.zeros((M, K // 2), dtype=torch.uint8)
        xc[:, 0] = one
        xs = torch.full((M, nb), 0x38, dtype=torch.uint8)
        wc = torch.zeros((N, K // 2), dtype=torch.uint8)
        wc[:, 0] = one
        ws = torch.full((N, nb), 0x38, dtype=torch.uint8)
        ws[:, 0] = sel
    for dt in (torch.float32, torch.bfloat16):
        y = gpu_linear(focus, xc, xs, np.float32(1.0), wc, ws, np.float32(1.0), dt)
        assert np.array_equal(y, np.broadcast_to(want, (M, N))), f"{side} {nb} {M} {dt}"


def test_linear_beyond_32bit_outputs(focus, orc):
    """Y [32770, 65540] (2^31 + 262,312 outputs, 4.3 GB of BF16) with K = 64:
    whole output rows on both sides of element 2^31 (row 32768 holds it) and
    the last row match the oracle within the bound."""
    M, N, K = 32770, 65540, 64
    xc, xs, wc, ws = operands(M, N, K, 13)
    s2x = np.full(M, 2.0 ** -9, dtype=np.float32)
    s2w = np.float32(1.5e-3)
    x = focus.Quantized(xc.to(DEV), xs.to(DEV), None, torch.from_numpy(s2x).to(DEV))
    w = focus.Quantized(wc.to(DEV), ws.to(DEV), None, torch.tensor([s2w], dtype=torch.float32, device=DEV))
    y = focus.nvfp4_linear(x, w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.array([0, 32767, 32768, 32769])
    ref, refabs = oracle_linear(orc, xc[idx].numpy(), xs[idx].numpy(), s2x[idx], wc.numpy(), ws.numpy(), s2w)
    got = y[torch.from_numpy(idx).to(DEV)].float().cpu().numpy().astype(np.float64)
    check_bound(got, ref, refabs, K, True, "Y past 2^31 outputs")


def test_linear_degenerate(focus):
    x = focus.Quantized(torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                        torch.zeros((5, 0), dtype=torch.uint8, device=DEV), None,
                        torch.ones(5, dtype=torch.float32, device=DEV))
    w = focus.Quantized(torch.zeros((3, 0), dtype=torch.uint8, device=DEV),
                        torch.zeros((3, 0), dtype=torch.uint8, device=DEV), None,
                        torch.ones(1, dtype=torch.float32, device=DEV))
    y = focus.nvfp4_linear(x, w, out_dtype=torch.float32, out=torch.full((5, 3), 7.0, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(y, torch.zeros((5, 3), device=DEV))  # K = 0: the empty sum


@pytest.mark.parametrize("N,K", sorted(set(synth.LLAMA_8B.layer_shapes())) + [(28672, 8192), (8192, 28672)],
                         ids=lambda v: str(v))
def test_linear_full_size_sampled(focus, orc, N, K):
    """8192 tokens through every 8B linear shape at full size (the launch the
    benchmark times); sampled rows and columns against the oracle."""
    M = 8192
    xc, xs = synth.nvfp4_operand(M, K, seed=7, tensor_id=42, device=DEV)
    wc, ws = synth.nvfp4_operand(N, K, seed=7, tensor_id=43, device=DEV)
    s2x = torch.rand(M, generator=synth.generator(7, 44, DEV), device=DEV) * 1e-3 + 1e-4
    s2w = torch.tensor([2.0e-4], device=DEV)
    y = focus.nvfp4_linear(focus.Quantized(xc, xs, None, s2x), focus.Quantized(wc, ws, None, s2w),
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N + K)
    ri = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    ci = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 62)]))
    ref, refabs = oracle_linear(orc, xc[ri].cpu().numpy(), xs[ri].cpu().numpy(), s2x[ri].cpu().numpy(),
                                wc[ci].cpu().numpy(), ws[ci].cpu().numpy(), np.float32(2.0e-4))
    got = y[torch.from_numpy(ri).to(DEV)][:, torch.from_numpy(ci).to(DEV)].float().cpu().numpy().astype(np.float64)
    check_bound(got, ref, refabs, K, True, f"8192 x {N} x {K}")


@pytest.mark.parametrize("M", [1, 16, 64, 128])
@pytest.mark.parametrize("N,K", sorted(set(synth.LLAMA_8B.layer_shapes() + synth.LLAMA_70B.layer_shapes())),
                         ids=lambda v: str(v))
def test_linear_few_tokens_full_size(focus, orc, M, N, K):
    """Decode-sized activations through every 8B linear shape at full size;
    all rows, sampled columns against the oracle."""
    xc, xs = synth.nvfp4_operand(M, K, seed=9, tensor_id=45, device=DEV)
    wc, ws = synth.nvfp4_operand(N, K, seed=9, tensor_id=46, device=DEV)
    s2x = torch.rand(M, generator=synth.generator(9, 47, DEV), device=DEV) * 1e-3 + 1e-4
    s2w = torch.tensor([3.0e-4], device=DEV)
    y = focus.nvfp4_linear(focus.Quantized(xc, xs, None, s2x), focus.Quantized(wc, ws, None, s2w),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    ci = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N + K + M).integers(0, N, 94)]))
    ref, refabs = oracle_linear(orc, xc.cpu().numpy(), xs.cpu().numpy(), s2x.cpu().numpy(), wc[ci].cpu().numpy(),
                                ws[ci].cpu().numpy(), np.float32(3.0e-4))
    got = y[:, torch.from_numpy(ci).to(DEV)].cpu().numpy().astype(np.float64)
    check_bound(got, ref, refabs, K, False, f"{M} x {N} x {K}")


def test_split_model_workspace(focus):
    """The split-k cost model on this GPU's compute units: outputs with enough
    tiles, or a single k-step, never split; few tiles with long rows do."""
    ws = focus.nvfp4_linear_workspace_bytes
    assert ws(8192, 14336, 4096) == 0                 # enough tiles: no split
    assert ws(2048, 1024, 4096) > 0 and ws(2048, 1024, 4096) % (2048 * 1024 * 4) == 0
    assert ws(16, 1024, 28672) > 0                    # few tokens, few columns, long rows
    assert ws(16, 4096, 64) == 0                      # one k-step: nothing to split
    assert ws(0, 16, 16) == 0 and ws(16, 16, 0) == 0


# members sharing one X: a layer's q, k, v (and gate, up) at small and full
# sizes; ragged N, K not a multiple of 256 (masked loads), M on both kernels
GROUPS = [(16, [4096, 1024, 1024], 4096), (1, [14336, 14336], 4096), (5, [17, 300, 1], 1040),
          (64, [520, 100, 33, 7, 1, 2, 3, 4, 5], 512), (128, [256, 130], 2064), (129, [130, 60], 192),
          (300, [520, 96], 1040), (16, [16000, 417], 512),  # two tiles through LDS, ragged member
          (64, [16000, 417], 512)]  # four tiles, ragged member


@pytest.mark.parametrize("M,Ns,K", GROUPS, ids=lambda v: str(v))
def test_linear_grouped_matches_oracle(focus, orc, M, Ns, K):
    """nvfp4_linear_grouped against the oracle for every member (within the
    bound; bit for bit where all partial sums are exact), FP32 and BF16
    output; nine members take two launches."""
    xc, xs = synth.nvfp4_operand(M, K, seed=M + K, tensor_id=48)
    rng = np.random.default_rng(M * 7 + K)
    s2x = (rng.uniform(0.5, 2.0, M) * 2.0 ** -9).astype(np.float32)
    ws = [synth.nvfp4_operand(N, K, seed=N + i, tensor_id=49) for i, N in enumerate(Ns)]
    s2w = [np.float32(3.0e-4 * (i + 1)) for i in range(len(Ns))]
    x = focus.Quantized(xc.to(DEV), xs.to(DEV), None, torch.from_numpy(s2x).to(DEV))
    wq = [focus.Quantized(c.to(DEV), s.to(DEV), None, torch.tensor([v], device=DEV)) for (c, s), v in zip(ws, s2w)]
    for dt in (torch.float32, torch.bfloat16):
        ys = focus.nvfp4_linear_grouped(x, wq, out_dtype=dt)
        torch.cuda.synchronize()
        for i, ((c, s), v) in enumerate(zip(ws, s2w)):
            ref, refabs = oracle_linear(orc, xc.numpy(), xs.numpy(), s2x, c.numpy(), s.numpy(), v)
            check_bound(ys[i].float().cpu().numpy().astype(np.float64), ref, refabs, K, dt == torch.bfloat16,
                        f"member {i} of {(M, Ns, K)} {dt}")
    # exact partial sums: all scales 1, power-of-two s2
    one_x = torch.full((M, K // 16), 0x38, dtype=torch.uint8)
    x1 = focus.Quantized(xc.to(DEV), one_x.to(DEV), None, torch.full((M,), 0.25, device=DEV))
    w1 = [focus.Quantized(c.to(DEV), torch.full((c.shape[0], K // 16), 0x38, dtype=torch.uint8, device=DEV), None,
                          torch.tensor([0.5], device=DEV)) for c, _ in ws]
    ys = focus.nvfp4_linear_grouped(x1, w1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, (c, _) in enumerate(ws):
        ref, _ = oracle_linear(orc, xc.numpy(), one_x.numpy(), np.full(M, 0.25, np.float32), c.numpy(),
                               np.full((c.shape[0], K // 16), 0x38, np.uint8), np.float32(0.5))
        assert np.array_equal(ys[i].cpu().numpy().astype(np.float64), ref), f"member {i} of {(M, Ns, K)}"


def test_linear_grouped_validation(focus):
    lib = focus._lib.lib()
    LW = focus._lib.LinearWeight
    FAKE = 0x10000
    g = lib.focus_nvfp4_linear_grouped
    good = LW(FAKE, FAKE, FAKE, 8, FAKE)
    assert g(FAKE, FAKE, FAKE, 1, 4, 64, (LW * 2)(good, LW(FAKE, FAKE, None, 8, FAKE)), 2, 0, None, 0,
             None) == 1   # a member's NULL s2, before any launch
    assert g(FAKE, FAKE, FAKE, 1, 4, 60, (LW * 1)(good), 1, 0, None, 0, None) == 2          # K % 16
    assert g(FAKE, FAKE, FAKE, 1, 4, 64, (LW * 1)(LW(FAKE + 4, FAKE, FAKE, 8, FAKE)), 1, 0, None, 0,
             None) == 3   # misaligned member codes
    assert g(FAKE, FAKE, FAKE, 1, 4, 64, None, 1, 0, None, 0, None) == 1
    assert g(FAKE, FAKE, FAKE, 1, 4, 64, (LW * 1)(good), -1, 0, None, 0, None) == 5
    assert g(FAKE, FAKE, FAKE, 1, 0, 64, (LW * 1)(good), 1, 0, None, 0, None) == 0           # M == 0: no-op
