"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by
element, on the same seeded inputs.  Runs on an MI355X only (marker gpu).

Sizes: the full single linear and per-token activation cases; ragged shapes
that span several 256-lane tiles with a partial tail; edge cases (zero
blocks, signed zeros, an all-zero tensor, extreme magnitudes, subnormal
scales, extreme logits); and every linear shape of the 8B and 70B weight
sets at full size, launched exactly as the benchmark launches them and
checked on sampled rows (plus the full tensor scale); the benchmark itself
checks every output of the whole 1B and 8B sets against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle_pins as pins
import parity
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def focus():
    import fp4_post_weight_amd as f
    f._lib.lib()  # raises if the library is not built: no fallback
    assert torch.cuda.is_available()
    return f


def np_bits(t):
    return synth.bits(t)


def run_weights(focus, w, m, q, dequant=True, s2=None):
    wd = w.to(DEV)
    md = None if m is None else m.to(DEV)
    qd = None if q is None else q.to(DEV)
    if s2 is None:
        s2d, amaxd = focus.tensor_scale(wd)
    else:
        s2d, amaxd = torch.tensor([s2], dtype=torch.float32, device=DEV), None
    res = focus.quantize(wd, md, qd, s2d, dequant=dequant)
    torch.cuda.synchronize()
    return (res.codes.cpu().numpy(), res.scales.cpu().numpy(),
            None if res.deq is None else np_bits(res.deq), np.float32(s2d.item()),
            None if amaxd is None else np.float32(amaxd.item()))


def check_case(focus, orc, w, m, q, dequant=True, label=""):
    wb = np_bits(w)
    mn = None if m is None else m.numpy()
    qn = None if q is None else q.numpy()
    codes, scales, deq, s2, amax = run_weights(focus, w, m, q, dequant)
    s2_o, amax_o = orc.tensor_scale(wb)
    assert s2.view(np.uint32) == s2_o.view(np.uint32), f"{label}: s2 {s2} vs {s2_o}"
    assert amax.view(np.uint32) == amax_o.view(np.uint32), label
    return parity.check_quantized(orc, wb, mn, qn, s2_o, codes, scales, deq, label=label)


# ---------------------------------------------------------------------------
# the single linear, ragged shapes, variants
# ---------------------------------------------------------------------------

def test_single_linear(focus, orc):
    w, m, q = synth.make_single()
    st = check_case(focus, orc, w, m, q, True, "single [256,1024]")
    assert st["code_mismatches"] == 0


RAGGED = [(1, 16), (3, 48), (7, 112), (33, 4112), (5, 2064), (129, 1040), (1, 65536 + 16)]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("variant", ["m_q_dq", "m_q", "q_only", "m_only", "plain_dq"])
def test_ragged_shapes(focus, orc, shape, variant):
    rows, cols = shape
    seed = rows * 7919 + cols
    w = synth.weights(shape, seed=seed, tensor_id=1, zero_block_p=0.02)
    m = synth.block_factor_lognormal((rows, cols // 16), seed=seed, tensor_id=2) \
        if "m" in variant.split("_") else None
    q = synth.logits((rows, cols // 8), seed=seed, tensor_id=3) if "q" in variant else None
    check_case(focus, orc, w, m, q, dequant=variant.endswith("dq"), label=f"{shape} {variant}")


def test_fixed_points_and_closed_forms(focus, orc):
    """The constructed blocks of the oracle pins, through the GPU."""
    rng = np.random.default_rng(21)
    sbytes, S, codes, wb = pins._fixed_point_case(rng, n_rows=111, nb=5)
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
    m2 = rng.integers(0, 2, (111, 5)).astype(bool)
    m = torch.from_numpy(np.where(m2, 2.0, 1.0).astype(np.float32))
    half = rng.integers(0, 2, (111, 10)).astype(bool)
    q = torch.from_numpy(np.where(half, 0.0, np.inf).astype(np.float32))
    for mm, qq in [(None, None), (m, None), (None, q), (m, q)]:
        g = run_weights(focus, w, mm, qq, True, s2=float(pins.S2_POW2))
        ref = orc.quantize(wb, None if mm is None else mm.numpy(), None if qq is None else qq.numpy(),
                           pins.S2_POW2, True)
        assert np.array_equal(g[0], ref[0]) and np.array_equal(g[1], ref[1])
        assert np.array_equal(g[2], ref[2])


def test_zero_blocks_and_signed_zeros(focus, orc):
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((40, 512)) * 0.02).astype(np.float32)
    wb = pins.torch_bf16_bits(x)
    wb[0, :] = 0
    wb[1, :] = 0x8000
    wb[2, 16:32] = 0x8000
    wb[3, ::2] = 0x8000
    wb[3, 1::2] = 0
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
    m = torch.ones((40, 32))
    m[5, 3] = 0.0
    q = synth.logits((40, 64), seed=3, tensor_id=0)
    st = check_case(focus, orc, w, m, q, True, "zero blocks")
    assert st["code_mismatches"] == 0


def test_all_zero_tensor(focus, orc):
    wb = np.zeros((8, 64), np.uint16)
    wb[2, 7] = 0x8000
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
    codes, scales, deq, s2, amax = run_weights(focus, w, None, synth.logits((8, 8), seed=1, tensor_id=0))
    assert s2 == 0 and amax == 0
    assert np.all(scales == 0x38)
    ref = orc.quantize(wb, None, None, np.float32(0))
    assert np.array_equal(codes, ref[0]) and np.array_equal(deq, ref[2])


def test_extreme_magnitudes(focus, orc):
    """Near-largest BF16 values, subnormal BF16 weights, mixed scales."""
    rng = np.random.default_rng(23)
    rows, cols = 64, 256
    e = rng.integers(-140, 127, (rows, cols)).astype(np.float64)
    x = (rng.standard_normal((rows, cols)) * np.exp2(e)).astype(np.float32)
    x[0, 0] = 3.3e38
    wb = pins.torch_bf16_bits(x)
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
    q = synth.logits((rows, cols // 8), seed=4, tensor_id=0)
    m = synth.block_factor_lognormal((rows, cols // 16), seed=4, tensor_id=1)
    check_case(focus, orc, w, m, q, True, "extreme magnitudes")


@pytest.mark.parametrize("amax_exp", [-133, -126, -120, -100])
def test_tiny_tensor_subnormal_scales(focus, orc, amax_exp):
    """amax near the bottom of the BF16 range: s2 and the denominators
    (S*sigmoid)*s2 are binary32 subnormals or underflow to 0 (the literal
    binary32 division path)."""
    rng = np.random.default_rng(100 - amax_exp)
    rows, cols = 16, 128
    x = (rng.uniform(-1, 1, (rows, cols)) * 2.0 ** amax_exp).astype(np.float32)
    wb = pins.torch_bf16_bits(x)
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
    q = torch.from_numpy(rng.uniform(-5, 20, (rows, cols // 8)).astype(np.float32))
    check_case(focus, orc, w, None, q, True, f"tiny 2^{amax_exp}")


def test_extreme_logits(focus, orc):
    rows, cols = 32, 512
    w = synth.weights((rows, cols), seed=5, tensor_id=1)
    vals = np.array([np.inf, 100.0, 17.0, 16.0, 6.0, 0.0, -0.0, -1.0, -10.0, -20.0, -40.0],
                    np.float32)
    rng = np.random.default_rng(24)
    q = torch.from_numpy(vals[rng.integers(0, len(vals), (rows, cols // 8))])
    check_case(focus, orc, w, None, q, True, "extreme logits")


# ---------------------------------------------------------------------------
# tensor scale, dequantize, round trip, determinism, streams
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("numel", [0, 1, 7, 8, 9, 15, 16, 17, 4093, 1_000_003, (1 << 22) + 5])
def test_tensor_scale_sizes(focus, orc, numel):
    rng = np.random.default_rng(numel)
    x = (rng.standard_normal(numel) * 0.02).astype(np.float32)
    if numel > 3:
        x[numel // 3] = -7.5  # the maximum magnitude is negative
    wb = pins.torch_bf16_bits(x)
    w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    s2, amax = focus.tensor_scale(w)
    s2_o, amax_o = orc.tensor_scale(wb)
    assert s2.item() == float(s2_o) and amax.item() == float(amax_o)


def test_dequantize_every_scale_byte(focus, orc):
    rows, cols = 254, 64
    rng = np.random.default_rng(25)
    codes = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    sb = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    scales = np.repeat(sb[:, None], cols // 16, axis=1)
    scales[:, 1] = sb[::-1]
    s2t = np.float32(0.0123)
    s2r = rng.uniform(1e-6, 3.0, rows).astype(np.float32)
    cd, sd = torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV)
    out_t = focus.dequantize(cd, sd, torch.tensor([s2t], device=DEV))
    out_r = focus.dequantize(cd, sd, torch.from_numpy(s2r).to(DEV), s2_per_row=True)
    assert np.array_equal(np_bits(out_t), orc.dequantize(codes, scales, s2t))
    assert np.array_equal(np_bits(out_r), orc.dequantize(codes, scales, s2r, s2_per_row=True))


def test_roundtrip_determinism_and_stream(focus, orc):
    w, m, q = synth.make_single(seed=7)
    wd, md, qd = w.to(DEV), m.to(DEV), q.to(DEV)
    r1 = focus.quantize(wd, md, qd, None, dequant=True)
    r2 = focus.quantize(wd, md, qd, None, dequant=True)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        r3 = focus.quantize(wd, md, qd, None, dequant=True)
        back = focus.dequantize(r3.codes, r3.scales, r3.s2)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    for r in (r2, r3):
        assert torch.equal(r.codes, r1.codes) and torch.equal(r.scales, r1.scales)
        assert torch.equal(r.deq.view(torch.int16), r1.deq.view(torch.int16))
    assert torch.equal(back.view(torch.int16), r1.deq.view(torch.int16))
    r4 = focus.quantize(wd, md, qd, r1.s2, dequant=False)
    assert r4.deq is None and torch.equal(r4.codes, r1.codes)


# ---------------------------------------------------------------------------
# per-token activations
# ---------------------------------------------------------------------------

def check_act(focus, orc, x, dequant, label):
    res = focus.quantize_act_per_token(x.to(DEV), dequant=dequant)
    torch.cuda.synchronize()
    xb = np_bits(x)
    c, s, s2, xd = parity.oracle_act_rows(orc, xb, dequant)
    assert np.array_equal(res.s2.cpu().numpy().view(np.uint32), s2.view(np.uint32)), label
    assert np.array_equal(res.scales.cpu().numpy(), s), label
    assert np.array_equal(res.codes.cpu().numpy(), c), label
    if dequant:
        assert np.array_equal(np_bits(res.deq), xd), label


def test_act_per_token_full(focus, orc):
    """The activation case: X [8192, 4096], N(0,1) with 2 % outlier channels."""
    check_act(focus, orc, synth.make_activations(), False, "act [8192,4096]")


# 5000 and 8197 tokens: workgroups take one or two rows in turn (the grid
# stops at 1024 workgroups below 8192 tokens, two rows per wavefront above)
@pytest.mark.parametrize("shape", [(1, 16), (5, 1024), (6, 2048), (7, 4096), (9, 8192), (3, 16400),
                                   (13, 48), (2, 4112), (5000, 4096), (8197, 1040)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_act_per_token_shapes(focus, orc, shape):
    x = synth.activations(shape, seed=shape[0] * 31 + shape[1], tensor_id=0)
    x[0, :16] = 0.0
    if shape[0] > 2:
        x[2] = 0.0  # an all-zero token: s2 = 0
    check_act(focus, orc, x, True, f"act {shape}")


# ---------------------------------------------------------------------------
# full-size linears, sampled rows
# ---------------------------------------------------------------------------

# every distinct linear shape of the 1B, 8B and 70B weight sets
FULL = [("1B", s) for s in sorted(set(synth.LLAMA_1B.layer_shapes()))] + \
       [("8B", s) for s in sorted(set(synth.LLAMA_8B.layer_shapes()))] + \
       [("70B", s) for s in sorted(set(synth.LLAMA_70B.layer_shapes()))]


@pytest.mark.parametrize("ws_name,shape", FULL, ids=lambda v: v if isinstance(v, str) else f"{v[0]}x{v[1]}")
@pytest.mark.parametrize("dequant", [False, True], ids=["codes", "codes+deq"])
def test_full_size_sampled(focus, orc, ws_name, shape, dequant):
    ws = {"1B": synth.LLAMA_1B, "8B": synth.LLAMA_8B, "70B": synth.LLAMA_70B}[ws_name]
    lin = next(l for l in ws.linears() if (l.rows, l.cols) == shape)
    w, m, q = synth.make_linear(ws, lin, device=DEV)
    s2d, amaxd = focus.tensor_scale(w)
    res = focus.quantize(w, m, q, s2d, dequant=dequant)
    torch.cuda.synchronize()
    rows, cols = shape
    rng = np.random.default_rng(rows + cols)
    idx = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 46)]))
    it = torch.from_numpy(idx).to(DEV)
    wb_full = np_bits(w)
    s2_o, amax_o = orc.tensor_scale(wb_full)
    assert s2d.item() == float(s2_o) and amaxd.item() == float(amax_o)
    wb = wb_full[idx]
    mn, qn = m[it].cpu().numpy(), q[it].cpu().numpy()
    st = parity.check_quantized(orc, wb, mn, qn, s2_o, res.codes[it].cpu().numpy(),
                                res.scales[it].cpu().numpy(),
                                np_bits(res.deq[it]) if dequant else None,
                                label=f"{ws_name} {shape}")
    print(f"{ws_name} {shape} dequant={dequant}: {st}", flush=True)


# ---------------------------------------------------------------------------
# one tensor past 32-bit offsets
# ---------------------------------------------------------------------------

BIG = (131075, 16384)  # 2^31 + 49,152 weights; W, w' and the dequantized copy 4.3 GB each


def test_beyond_32bit_offsets(focus, orc):
    """One linear whose element offsets pass 2^31 and whose W, w' and
    dequantized bytes pass 2^32 (row 131072 starts at element 2^31): s2 of
    the whole tensor equals the oracle's, rows on both sides of the boundary
    and the last rows match the oracle, the codes-only call gives the same
    codes and scales as the call with w', and the stand-alone dequantize
    equals the fused w' everywhere."""
    rows, cols = BIG
    w = synth.weights(BIG, seed=7, tensor_id=900, device=DEV)
    m = synth.block_factor_lognormal((rows, cols // 16), seed=7, tensor_id=901, device=DEV)
    q = synth.logits((rows, cols // 8), seed=7, tensor_id=902, device=DEV)
    s2d, amaxd = focus.tensor_scale(w)
    res = focus.quantize(w, m, q, s2d, dequant=True)
    only = focus.quantize(w, m, q, s2d, dequant=False)
    assert torch.equal(only.codes, res.codes) and torch.equal(only.scales, res.scales)
    del only
    deq = focus.dequantize(res.codes, res.scales, s2d)
    assert torch.equal(deq.view(torch.int16), res.deq.view(torch.int16))
    del deq
    torch.cuda.synchronize()
    wb = np_bits(w)
    s2_o, amax_o = orc.tensor_scale(wb)
    assert s2d.item() == float(s2_o) and amaxd.item() == float(amax_o)
    rng = np.random.default_rng(11)
    idx = np.unique(np.concatenate([[0, 65535, 65536, 131070, 131071, 131072, 131073, rows - 1],
                                    rng.integers(0, rows, 24)]))
    it = torch.from_numpy(idx).to(DEV)
    st = parity.check_quantized(orc, wb[idx], m[it].cpu().numpy(), q[it].cpu().numpy(), s2_o,
                                res.codes[it].cpu().numpy(), res.scales[it].cpu().numpy(),
                                np_bits(res.deq[it]), label=f"{BIG}")
    print(f"{BIG}: {st}", flush=True)


def test_act_beyond_32bit_offsets(focus, orc):
    """Per-token activations X [262147, 8192] (2^31 + 24,576 elements): the
    tokens past element 2^31 match the oracle."""
    t, h = 262147, 8192
    x = synth.activations((t, h), seed=5, tensor_id=903, device=DEV)
    res = focus.quantize_act_per_token(x, dequant=True)
    torch.cuda.synchronize()
    idx = np.array([0, 131071, 262143, 262144, 262145, t - 1])
    it = torch.from_numpy(idx).to(DEV)
    xb = np_bits(x[it])
    c, s, s2, xd = parity.oracle_act_rows(orc, xb, True)
    assert np.array_equal(res.s2[it].cpu().numpy().view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(res.scales[it].cpu().numpy(), s)
    assert np.array_equal(res.codes[it].cpu().numpy(), c)
    assert np.array_equal(np_bits(res.deq[it]), xd)


# ---------------------------------------------------------------------------
# batched calls: identical to the single calls, and to the oracle
# ---------------------------------------------------------------------------

def _mixed_set(n, seed):
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(1, 70)), 16 * int(rng.integers(1, 90))) for _ in range(n)]
    shapes[3] = (0, 64)          # empty
    shapes[5] = (300, 4096)      # several tiles
    items = []
    for i, (r, c) in enumerate(shapes):
        w = synth.weights((r, c), seed=seed, tensor_id=4 * i, zero_block_p=0.01).to(DEV)
        m = synth.block_factor_lognormal((r, c // 16), seed=seed, tensor_id=4 * i + 1).to(DEV) \
            if i % 3 else None
        q = synth.logits((r, c // 8), seed=seed, tensor_id=4 * i + 2).to(DEV) if i % 4 else None
        items.append((w, m, q))
    return items


@pytest.mark.parametrize("n", [1, 7, 32, 33, 70])
def test_batched_calls_match_single_calls(focus, orc, n):
    items = _mixed_set(max(n, 6), seed=900 + n)[:n] if n >= 6 else _mixed_set(6, 900 + n)[:n]
    ws = [w for w, _, _ in items]
    ts = focus.tensor_scale_many(ws)
    # alternate the dequant flag to split the batch into several runs
    deq_flags = [bool(i % 5) for i in range(n)]
    outs = []
    for i, (w, m, q) in enumerate(items):
        r, c = w.shape
        outs.append(focus.Quantized(torch.empty((r, c // 2), dtype=torch.uint8, device=DEV),
                                    torch.empty((r, c // 16), dtype=torch.uint8, device=DEV),
                                    torch.empty((r, c), dtype=torch.bfloat16, device=DEV) if deq_flags[i] else None,
                                    ts.s2[i]))
    qb = focus.quantize_many(ws, [m for _, m, _ in items], [q for _, _, q in items],
                             [ts.s2[i] for i in range(n)], outs=outs, dequant=True)
    dq = focus.dequantize_many([o.codes for o in qb.outs], [o.scales for o in qb.outs],
                               [ts.s2[i] for i in range(n)])
    torch.cuda.synchronize()
    for i, (w, m, q) in enumerate(items):
        s2, amax = focus.tensor_scale(w)
        single = focus.quantize(w, m, q, s2, dequant=deq_flags[i])
        torch.cuda.synchronize()
        assert ts.s2[i].item() == s2.item() and ts.amax[i].item() == amax.item()
        assert torch.equal(qb.outs[i].codes, single.codes), i
        assert torch.equal(qb.outs[i].scales, single.scales), i
        if deq_flags[i]:
            assert torch.equal(qb.outs[i].deq.view(torch.int16), single.deq.view(torch.int16)), i
            assert torch.equal(dq.outs[i].view(torch.int16), single.deq.view(torch.int16)), i
        if i < 8 and w.numel():
            wb = np_bits(w)
            s2_o, _ = orc.tensor_scale(wb)
            parity.check_quantized(orc, wb, None if m is None else m.cpu().numpy(),
                                   None if q is None else q.cpu().numpy(), s2_o,
                                   single.codes.cpu().numpy(), single.scales.cpu().numpy(),
                                   np_bits(single.deq) if deq_flags[i] else None, label=f"batch item {i}")


def test_tensor_scale_many_sizes(focus, orc):
    sizes = [0, 1, 7, 8, 9, 4093, 65536 * 8 + 3, 16, 1_000_003] * 5
    rng = np.random.default_rng(31)
    host, ws = [], []
    for k, n in enumerate(sizes):
        x = (rng.standard_normal(n) * (k + 1)).astype(np.float32)
        wb = pins.torch_bf16_bits(x)
        host.append(wb)
        ws.append(torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16).to(DEV))
    ts = focus.tensor_scale_many(ws)
    torch.cuda.synchronize()
    for k, wb in enumerate(host):
        s2_o, amax_o = orc.tensor_scale(wb)
        assert ts.s2[k].item() == float(s2_o) and ts.amax[k].item() == float(amax_o), k


def test_dequantize_many_per_row_mix(focus, orc):
    rng = np.random.default_rng(32)
    codes, scales, s2s, flags, host = [], [], [], [], []
    for k in range(40):
        r, c = int(rng.integers(1, 50)), 16 * int(rng.integers(1, 40))
        cd = rng.integers(0, 256, (r, c // 2)).astype(np.uint8)
        sc = rng.integers(0x08, 0x7F, (r, c // 16)).astype(np.uint8)
        pr = bool(k % 2)
        s2 = rng.uniform(1e-5, 1.0, r if pr else 1).astype(np.float32)
        host.append((cd, sc, s2, pr))
        codes.append(torch.from_numpy(cd).to(DEV))
        scales.append(torch.from_numpy(sc).to(DEV))
        s2s.append(torch.from_numpy(s2).to(DEV))
        flags.append(pr)
    dq = focus.dequantize_many(codes, scales, s2s, s2_per_row=flags)
    torch.cuda.synchronize()
    for k, (cd, sc, s2, pr) in enumerate(host):
        assert np.array_equal(np_bits(dq.outs[k]), orc.dequantize(cd, sc, s2, s2_per_row=pr)), k


# ---------------------------------------------------------------------------
# FourOverSix (weights per tensor, activations per token)
# ---------------------------------------------------------------------------

def run_fo6(focus, wb, s2=None, dequant=True):
    w = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    s2d = None if s2 is None else torch.tensor([s2], dtype=torch.float32, device=DEV)
    res = focus.quantize_fo6(w, s2d, dequant=dequant)
    torch.cuda.synchronize()
    return (res.codes.cpu().numpy(), res.scales.cpu().numpy(),
            None if res.deq is None else np_bits(res.deq), np.float32(res.s2.item()))


def check_fo6(focus, orc, wb, dequant=True, s2=None, label=""):
    codes, scales, deq, s2g = run_fo6(focus, wb, s2, dequant)
    if s2 is None:
        s2_o, _ = orc.tensor_scale(wb)
        assert s2g == s2_o, label
    else:
        s2_o = np.float32(s2)
    c, sc, d = orc.fo6_quantize(wb, s2_o, dequant=dequant)
    assert np.array_equal(scales, sc), f"{label}: {np.count_nonzero(scales != sc)} scale bytes differ"
    assert np.array_equal(codes, c), f"{label}: {np.count_nonzero(codes != c)} code bytes differ"
    if dequant:
        assert np.array_equal(deq, d), label
    return np.count_nonzero(sc != orc.quantize(wb, None, None, s2_o, dequant=False)[1])


def test_fo6_single_linear_and_ragged(focus, orc):
    w, _, _ = synth.make_single()
    n4 = check_fo6(focus, orc, np_bits(w), label="fo6 single [256,1024]")
    assert n4 > 1000  # a large share of Gaussian blocks prefer the 4-candidate
    for shape in RAGGED:
        wr = synth.weights(shape, seed=shape[0] + 7 * shape[1], tensor_id=9, zero_block_p=0.02)
        check_fo6(focus, orc, np_bits(wr), dequant=shape[0] % 2 == 1, label=f"fo6 {shape}")


def test_fo6_constructed_cases(focus, orc):
    rng = np.random.default_rng(70)
    _, _, wb4, _ = pins._fo6_four_case(rng)
    check_fo6(focus, orc, wb4, s2=float(pins.S2_POW2), label="fo6 four fixed points")
    _, _, _, wb6 = pins._fixed_point_case(rng, n_rows=119, nb=3)
    check_fo6(focus, orc, wb6, s2=float(pins.S2_POW2), label="fo6 six fixed points")
    wz = np.zeros((4, 64), np.uint16)
    wz[1, 3] = 0x8000
    check_fo6(focus, orc, wz, label="fo6 all zero")


def test_fo6_extreme_magnitudes(focus, orc):
    rng = np.random.default_rng(71)
    e = rng.integers(-140, 127, (64, 256)).astype(np.float64)
    x = (rng.standard_normal((64, 256)) * np.exp2(e)).astype(np.float32)
    x[0, 0] = 3.3e38
    check_fo6(focus, orc, pins.torch_bf16_bits(x), label="fo6 extreme")
    for amax_exp in (-133, -120):
        y = (rng.uniform(-1, 1, (16, 128)) * 2.0 ** amax_exp).astype(np.float32)
        check_fo6(focus, orc, pins.torch_bf16_bits(y), label=f"fo6 tiny 2^{amax_exp}")


def _fo6_errors_f32(blocks, s2):
    """Test-side search aid (never an expected value): numpy binary32
    emulation of both FourOverSix candidates' error sums and of the kernel's
    cheap estimate, used only to pick blocks whose decision is close."""
    f32 = np.float32
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.abs(blocks).max(1)
    out = {}
    for k in (6, 4):
        t = (a / f32(f32(k) * s2)).astype(f32)
        t = np.clip(np.where(t == 0, f32(1), t), f32(2 ** -6), f32(448))
        u = t.view(np.uint32).astype(np.uint64)
        S = (((u + 0x7FFFF + ((u >> 20) & 1)) >> 20) << 20).astype(np.uint32).view(f32)
        d = (S * s2).astype(f32)
        x = (blocks.astype(np.float64) / d[:, None]).astype(f32)
        dist = np.abs(np.minimum(np.abs(x), 6)[..., None].astype(np.float64) - grid)
        c = (np.sign(x) * grid[np.argmin(dist + (np.arange(8) % 2) * 1e-12, axis=-1)]).astype(f32)
        v = ((c * S[:, None]).astype(f32) * s2).astype(f32)
        q = ((blocks - v).astype(f32) ** 2).astype(f32)
        E = np.zeros(len(blocks), f32)
        for i in range(16):
            E = (E + q[:, i]).astype(f32)
        out[k] = (E, S, d)
    return out


def test_fo6_near_ties_take_the_exact_path(focus, orc):
    """Blocks whose two candidates' exact errors are within the estimate's
    margin (relative gap below 2^-16) or exactly equal with different scales
    are decided by the exact sums; searched among 2 M Gaussian blocks, with
    outlier blocks (one large element, the rest small) for exact ties, and
    checked bit for bit against the oracle."""
    rng = np.random.default_rng(2024)
    s2 = np.float32(0.02 * 4.5 / 2688)
    blocks = pins.torch_bf16_bits((rng.standard_normal((1 << 21, 16)) * 0.02).astype(np.float32))
    vals = (blocks.astype(np.uint32) << 16).view(np.float32)
    e = _fo6_errors_f32(vals, s2)
    (E6, S6, _), (E4, S4, _) = e[6], e[4]
    gap = np.abs(E4 - E6) / np.maximum(E6, 1e-30)
    near = np.nonzero((gap < 2.0 ** -16) & (S4 != S6))[0]
    assert len(near) >= 8, len(near)
    # outlier blocks: one element of about 1200 s2 (block scale t6 near 200,
    # so S4 = 1.5 S6 whenever S6 is 128, 160 or 192 times a power of two) and
    # the others too small for a nonzero code: both candidates dequantize to
    # the same values, an exact tie
    ob = (rng.standard_normal((4096, 16)) * 3e-4).astype(np.float32)
    ob[np.arange(4096), rng.integers(0, 16, 4096)] = rng.uniform(0.03, 0.05, 4096) * np.sign(
        rng.standard_normal(4096))
    ob = pins.torch_bf16_bits(ob)
    ov = (ob.astype(np.uint32) << 16).view(np.float32)
    eo = _fo6_errors_f32(ov, s2)
    ties = np.nonzero((eo[4][0] == eo[6][0]) & (eo[4][1] != eo[6][1]))[0]
    assert len(ties) >= 8, len(ties)
    sel = np.concatenate([blocks[near], ob[ties]])
    sel = np.concatenate([sel, np.zeros(((-len(sel)) % 8, 16), np.uint16)])
    wb = np.ascontiguousarray(sel.reshape(-1, 128))
    check_fo6(focus, orc, wb, s2=float(s2), label=f"fo6 near ties ({len(near)} close, {len(ties)} exact)")
    # the same blocks as per-token activations rows (per-row s2)
    xb = np.ascontiguousarray(sel[: (len(sel) // 16) * 16].reshape(-1, 256))
    x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16)
    check_act_fo6(focus, orc, x, True, "fo6 act near ties")


@pytest.mark.parametrize("s2", [2.0 ** -54, 2.0 ** -54 * 1.5, 2.0 ** 47 * 1.9, 2.0 ** 48, 2.0 ** -55, 2.0 ** 49],
                         ids=lambda v: f"{v:.3g}")
def test_fo6_estimate_range_boundaries(focus, orc, s2):
    """s2 at and just beyond the ends of the range in which the cheap
    estimate decides (below and above it every block takes the exact sums)."""
    rng = np.random.default_rng(int(np.log2(s2) * 10) & 0xFFFF)
    x = (rng.standard_normal((64, 256)) * (s2 * 2688 / 4.5)).astype(np.float32)
    check_fo6(focus, orc, pins.torch_bf16_bits(x), s2=float(np.float32(s2)), label=f"fo6 s2={s2:.3g}")


@pytest.mark.parametrize("shape", sorted(set(synth.LLAMA_8B.layer_shapes())), ids=lambda s: f"{s[0]}x{s[1]}")
def test_fo6_full_size_sampled(focus, orc, shape):
    lin = next(l for l in synth.LLAMA_8B.linears() if (l.rows, l.cols) == shape)
    w, _, _ = synth.make_linear(synth.LLAMA_8B, lin, device=DEV, with_m=False, with_q=False)
    res = focus.quantize_fo6(w, dequant=True)
    torch.cuda.synchronize()
    wb = np_bits(w)
    s2_o, _ = orc.tensor_scale(wb)
    assert res.s2.item() == float(s2_o)
    rows = shape[0]
    idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(rows).integers(0, rows, 30)]))
    it = torch.from_numpy(idx).to(DEV)
    c, sc, d = orc.fo6_quantize(wb[idx], s2_o)
    assert np.array_equal(res.scales[it].cpu().numpy(), sc)
    assert np.array_equal(res.codes[it].cpu().numpy(), c)
    assert np.array_equal(np_bits(res.deq[it]), d)


def check_act_fo6(focus, orc, x, dequant, label):
    res = focus.quantize_act_per_token_fo6(x.to(DEV), dequant=dequant)
    torch.cuda.synchronize()
    xb = np_bits(x)
    rows = xb.shape[0]
    n = parity.threads()
    if rows >= 2 * n:
        from concurrent.futures import ThreadPoolExecutor
        bounds = np.linspace(0, rows, n + 1).astype(int)
        with ThreadPoolExecutor(n) as ex:
            parts = list(ex.map(lambda i: orc.fo6_quantize_act_per_token(xb[bounds[i]:bounds[i + 1]], dequant),
                                range(n)))
        c = np.concatenate([p[0] for p in parts])
        s = np.concatenate([p[1] for p in parts])
        s2 = np.concatenate([p[2] for p in parts])
        xd = np.concatenate([p[3] for p in parts]) if dequant else None
    else:
        c, s, s2, xd = orc.fo6_quantize_act_per_token(xb, dequant)
    assert np.array_equal(res.s2.cpu().numpy().view(np.uint32), s2.view(np.uint32)), label
    assert np.array_equal(res.scales.cpu().numpy(), s), label
    assert np.array_equal(res.codes.cpu().numpy(), c), label
    if dequant:
        assert np.array_equal(np_bits(res.deq), xd), label


def test_fo6_act_full(focus, orc):
    check_act_fo6(focus, orc, synth.make_activations(), False, "fo6 act [8192,4096]")


@pytest.mark.parametrize("shape", [(1, 16), (5, 1024), (6, 2048), (7, 4096), (9, 8192), (3, 16400)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_fo6_act_shapes(focus, orc, shape):
    x = synth.activations(shape, seed=shape[0] * 13 + shape[1], tensor_id=2)
    if shape[0] > 2:
        x[2] = 0.0
    check_act_fo6(focus, orc, x, True, f"fo6 act {shape}")


def test_fo6_many_matches_single(focus, orc):
    items = _mixed_set(40, seed=77)
    ws = [w for w, _, _ in items]
    ts = focus.tensor_scale_many(ws)
    b = focus.quantize_fo6_many(ws, [ts.s2[i] for i in range(len(ws))], dequant=True)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        single = focus.quantize_fo6(w, ts.s2[i], dequant=True)
        torch.cuda.synchronize()
        assert torch.equal(b.outs[i].codes, single.codes) and torch.equal(b.outs[i].scales, single.scales)
        assert torch.equal(b.outs[i].deq.view(torch.int16), single.deq.view(torch.int16))
    # the codes-only kernel (a tile size of its own) on the same batch: the
    # same codes and scales, and the oracle's on a few members
    bn = focus.quantize_fo6_many(ws, [ts.s2[i] for i in range(len(ws))], dequant=False)
    torch.cuda.synchronize()
    for i in range(len(ws)):
        assert torch.equal(bn.outs[i].codes, b.outs[i].codes), i
        assert torch.equal(bn.outs[i].scales, b.outs[i].scales), i
    for i in (0, 5, len(ws) - 1):
        c, sc, _ = orc.fo6_quantize(np_bits(ws[i].cpu()), np.float32(ts.s2[i].item()), dequant=False)
        assert np.array_equal(bn.outs[i].codes.cpu().numpy(), c), i
        assert np.array_equal(bn.outs[i].scales.cpu().numpy(), sc), i


# ---------------------------------------------------------------------------
# FOCUS on MXFP4
# ---------------------------------------------------------------------------

def run_mx(focus, wb, m=None, q=None, dequant=True):
    w = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    md = None if m is None else torch.from_numpy(np.ascontiguousarray(m)).to(DEV)
    qd = None if q is None else torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    res = focus.quantize_mx(w, md, qd, dequant=dequant)
    torch.cuda.synchronize()
    back = focus.dequantize_mx(res.codes, res.scales)
    torch.cuda.synchronize()
    return (res.codes.cpu().numpy(), res.scales.cpu().numpy(),
            None if res.deq is None else np_bits(res.deq), np_bits(back))


def check_mx(focus, orc, wb, m=None, q=None, dequant=True, label=""):
    codes, scales, deq, back = run_mx(focus, wb, m, q, dequant)
    c, s, d = orc.mx_quantize(wb, m, q, dequant=True)
    assert np.array_equal(scales, s), f"{label}: {np.count_nonzero(scales != s)} scale bytes differ"
    nbad = np.count_nonzero(parity.unpack(codes) != parity.unpack(c))
    assert nbad <= int(1e-6 * wb.size), f"{label}: {nbad} codes differ"
    if nbad == 0:
        if dequant:
            assert np.array_equal(deq, d), label
        assert np.array_equal(back, d), label
    return nbad


def test_mx_constructed_cases(focus, orc):
    rng = np.random.default_rng(90)
    sb, codes, wb = pins._mx_fixed_case(rng)
    assert check_mx(focus, orc, wb, label="mx fixed points") == 0
    m = np.where(rng.integers(0, 2, (wb.shape[0], wb.shape[1] // 32)) == 1, 2.0, 1.0).astype(np.float32)
    qv = np.where(rng.integers(0, 2, (wb.shape[0], wb.shape[1] // 8)) == 1, 0.0, np.inf).astype(np.float32)
    assert check_mx(focus, orc, wb, m, qv, label="mx m and q maps") == 0
    wz = np.zeros((4, 64), np.uint16)
    wz[1, 40] = 0x8000
    assert check_mx(focus, orc, wz, label="mx zeros") == 0


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (7, 4128), (33, 2080), (129, 1056)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("variant", ["m_q_dq", "m_q", "q_only", "plain_dq"])
def test_mx_ragged(focus, orc, shape, variant):
    rows, cols = shape
    seed = rows * 31 + cols
    wb = np_bits(synth.weights(shape, seed=seed, tensor_id=11, zero_block_p=0.02))
    m = synth.block_factor_lognormal((rows, cols // 32), seed=seed, tensor_id=12).numpy() \
        if "m" in variant.split("_") else None
    q = synth.logits((rows, cols // 8), seed=seed, tensor_id=13).numpy() if "q" in variant else None
    check_mx(focus, orc, wb, m, q, dequant=variant.endswith("dq"), label=f"mx {shape} {variant}")


def test_mx_extreme(focus, orc):
    rng = np.random.default_rng(91)
    e = rng.integers(-140, 127, (32, 256)).astype(np.float64)
    x = (rng.standard_normal((32, 256)) * np.exp2(e)).astype(np.float32)
    x[0, 0] = 3.3e38
    q = rng.uniform(-20, 30, (32, 32)).astype(np.float32)
    m = np.exp(rng.standard_normal((32, 8)) * 3).astype(np.float32)
    check_mx(focus, orc, pins.torch_bf16_bits(x), m, q, label="mx extreme")


@pytest.mark.parametrize("shape", sorted(set(synth.LLAMA_8B.layer_shapes())), ids=lambda s: f"{s[0]}x{s[1]}")
def test_mx_full_size_sampled(focus, orc, shape):
    rows, cols = shape
    lin = next(l for l in synth.LLAMA_8B.linears() if (l.rows, l.cols) == shape)
    w = synth.weights(shape, seed=42, tensor_id=lin.tid(0), device=DEV)
    m = synth.block_factor_lognormal((rows, cols // 32), seed=42, tensor_id=lin.tid(1), device=DEV)
    q = synth.logits((rows, cols // 8), seed=42, tensor_id=lin.tid(2), device=DEV)
    res = focus.quantize_mx(w, m, q, dequant=True)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(rows).integers(0, rows, 30)]))
    it = torch.from_numpy(idx).to(DEV)
    c, s, d = orc.mx_quantize(np_bits(w[it]), m[it].cpu().numpy(), q[it].cpu().numpy())
    assert np.array_equal(res.scales[it].cpu().numpy(), s)
    gc = parity.unpack(res.codes[it].cpu().numpy())
    nbad = np.count_nonzero(gc != parity.unpack(c))
    assert nbad <= int(1e-6 * gc.size)
    if nbad == 0:
        assert np.array_equal(np_bits(res.deq[it]), d)


def test_mx_many_matches_single(focus, orc):
    rng = np.random.default_rng(92)
    ws, ms, qs = [], [], []
    for i in range(37):
        r, c = int(rng.integers(1, 60)), 32 * int(rng.integers(1, 40))
        ws.append(synth.weights((r, c), seed=i, tensor_id=14).to(DEV))
        ms.append(synth.block_factor_lognormal((r, c // 32), seed=i, tensor_id=15).to(DEV) if i % 3 else None)
        qs.append(synth.logits((r, c // 8), seed=i, tensor_id=16).to(DEV) if i % 4 else None)
    b = focus.quantize_mx_many(ws, ms, qs, dequant=True)
    torch.cuda.synchronize()
    for i in range(37):
        single = focus.quantize_mx(ws[i], ms[i], qs[i], dequant=True)
        torch.cuda.synchronize()
        assert torch.equal(b.outs[i].codes, single.codes) and torch.equal(b.outs[i].scales, single.scales)
        assert torch.equal(b.outs[i].deq.view(torch.int16), single.deq.view(torch.int16))


# ---------------------------------------------------------------------------
# FlipQuant MixFP4 (per-tile E0M3 / E2M1-FourOverSix)
# ---------------------------------------------------------------------------

def run_mix(focus, wb, tmap, th, tw, s2=None, dequant=True):
    w = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    md = torch.from_numpy(np.ascontiguousarray(tmap, dtype=np.uint8)).to(DEV)
    s2d = None if s2 is None else torch.tensor([s2], dtype=torch.float32, device=DEV)
    res = focus.quantize_mixfp4(w, md, th, tw, s2d, dequant=dequant)
    torch.cuda.synchronize()
    return (res.codes.cpu().numpy(), res.scales.cpu().numpy(),
            None if res.deq is None else np_bits(res.deq), np.float32(res.s2.item()))


def check_mix(focus, orc, wb, tmap, th, tw, dequant=True, s2=None, label=""):
    codes, scales, deq, s2g = run_mix(focus, wb, tmap, th, tw, s2, dequant)
    if s2 is None:
        s2_o, _ = orc.tensor_scale(wb)
        assert s2g == s2_o, label
    else:
        s2_o = np.float32(s2)
    c, sc, d = orc.mixfp4_quantize(wb, s2_o, tmap, th, tw, dequant=dequant)
    assert np.array_equal(scales, sc), f"{label}: {np.count_nonzero(scales != sc)} scale bytes differ"
    assert np.array_equal(codes, c), f"{label}: {np.count_nonzero(codes != c)} code bytes differ"
    if dequant:
        assert np.array_equal(deq, d), f"{label}: {np.count_nonzero(deq != d)} w' values differ"


MIX_CASES = [((256, 1024), (8, 64)), ((256, 1024), (16, 64)), ((512, 1024), (256, 64)),
             ((24, 1088), (8, 64)), ((3, 48), (3, 48)), ((7, 112), (1, 16)), ((33, 4112), (11, 16)),
             ((129, 1040), (43, 208)), ((1, 65536 + 64), (1, 64))]


@pytest.mark.parametrize("shape,tile", MIX_CASES, ids=lambda v: f"{v[0]}x{v[1]}")
def test_mixfp4_maps(focus, orc, shape, tile):
    """Random maps at a high E0M3 share and at the page's share; full and
    odd tilings (the division by blocks per row, tile rows and tile columns
    in blocks at several divisors), partial last launch tiles."""
    rows, cols = shape
    w = synth.weights(shape, seed=rows + 3 * cols, tensor_id=21, zero_block_p=0.02)
    wb = np_bits(w)
    for i, frac in enumerate((0.4, synth.MIXFP4_FRAC.get(tile, 0.02))):
        tmap = synth.tile_map(rows, cols, tile, frac=frac, seed=rows + i, tensor_id=22).numpy()
        check_mix(focus, orc, wb, tmap, tile[0], tile[1], dequant=(i == 0) or rows % 2 == 1,
                  label=f"mix {shape} tile {tile} frac {frac:.4f}")


def test_mixfp4_constructed_cases(focus, orc):
    rng = np.random.default_rng(97)
    sb, codes, wb = pins._e0m3_fixed_case(rng, rows=24, nb=8)
    check_mix(focus, orc, wb, np.ones((3, 2), np.uint8), 8, 64, s2=float(pins.S2_POW2), label="e0m3 fixed points")
    # the GPU reproduces the fixed points themselves
    c, s, d, _ = run_mix(focus, wb, np.ones((3, 2), np.uint8), 8, 64, s2=float(pins.S2_POW2))
    assert np.array_equal(s, sb) and np.array_equal(parity.unpack(c), codes) and np.array_equal(d, wb)
    # all-clear map: FourOverSix bit for bit
    w, _, _ = synth.make_single()
    wb1 = np_bits(w)
    c0, s0, d0, _ = run_mix(focus, wb1, np.zeros((32, 16), np.uint8), 8, 64)
    f = focus.quantize_fo6(w.to(DEV), dequant=True)
    torch.cuda.synchronize()
    assert np.array_equal(c0, f.codes.cpu().numpy()) and np.array_equal(s0, f.scales.cpu().numpy())
    assert np.array_equal(d0, np_bits(f.deq))
    # all-zero tensor and signed zeros
    wz = np.zeros((16, 128), np.uint16)
    wz[1, 3] = 0x8000
    check_mix(focus, orc, wz, np.array([[1, 0], [0, 1]], np.uint8), 8, 64, label="mix all zero")


def test_mixfp4_extreme_magnitudes(focus, orc):
    rng = np.random.default_rng(98)
    e = rng.integers(-140, 127, (64, 256)).astype(np.float64)
    x = (rng.standard_normal((64, 256)) * np.exp2(e)).astype(np.float32)
    x[0, 0] = 3.3e38
    tmap = (rng.random((8, 4)) < 0.5).astype(np.uint8)
    check_mix(focus, orc, pins.torch_bf16_bits(x), tmap, 8, 64, label="mix extreme")
    for amax_exp in (-133, -120):
        y = (rng.uniform(-1, 1, (16, 128)) * 2.0 ** amax_exp).astype(np.float32)
        check_mix(focus, orc, pins.torch_bf16_bits(y), np.array([[1, 0], [0, 1]], np.uint8), 8, 64,
                  label=f"mix tiny 2^{amax_exp}")


@pytest.mark.parametrize("tile", [(8, 64), (16, 64), (256, 64)], ids=lambda t: f"{t[0]}x{t[1]}")
def test_mixfp4_full_size_sampled(focus, orc, tile):
    """Every 8B linear shape at full size with a map at the page's E0M3 share,
    launched batched as the benchmark launches them; sampled rows checked
    (row i against its map row, i.e. the oracle with one-row tiles)."""
    shapes = sorted(set(synth.LLAMA_8B.layer_shapes()))
    ws, maps = [], []
    for k, (rows, cols) in enumerate(shapes):
        lin = next(l for l in synth.LLAMA_8B.linears() if (l.rows, l.cols) == (rows, cols))
        w, _, _ = synth.make_linear(synth.LLAMA_8B, lin, device=DEV, with_m=False, with_q=False)
        ws.append(w)
        maps.append(synth.tile_map(rows, cols, tile, frac=synth.MIXFP4_FRAC[tile], seed=k, tensor_id=23,
                                   device=DEV))
    ts = focus.tensor_scale_many(ws)
    b = focus.quantize_mixfp4_many(ws, maps, [tile] * len(ws), [ts.s2[i] for i in range(len(ws))], dequant=True)
    torch.cuda.synchronize()
    for k, w in enumerate(ws):
        rows = w.shape[0]
        wb = np_bits(w)
        s2_o, _ = orc.tensor_scale(wb)
        assert ts.s2[k].item() == float(s2_o)
        idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(rows + k).integers(0, rows, 12)]))
        it = torch.from_numpy(idx).to(DEV)
        mrows = maps[k].cpu().numpy()[idx // tile[0]]
        c, sc, d = orc.mixfp4_quantize(wb[idx], s2_o, mrows, 1, tile[1])
        o = b.outs[k]
        assert np.array_equal(o.scales[it].cpu().numpy(), sc)
        assert np.array_equal(o.codes[it].cpu().numpy(), c)
        assert np.array_equal(np_bits(o.deq[it]), d)


def test_mixfp4_many_matches_single(focus, orc):
    rng = np.random.default_rng(99)
    ws, maps, tiles = [], [], []
    for i in range(37):
        th, tw = int(rng.integers(1, 9)), 16 * int(rng.integers(1, 5))
        r, c = th * int(rng.integers(1, 8)), tw * int(rng.integers(1, 20))
        ws.append(synth.weights((r, c), seed=i, tensor_id=24).to(DEV))
        maps.append(synth.tile_map(r, c, (th, tw), frac=0.3, seed=i, tensor_id=25, device=DEV))
        tiles.append((th, tw))
    ts = focus.tensor_scale_many(ws)
    s2s = [ts.s2[i] for i in range(37)]
    b = focus.quantize_mixfp4_many(ws, maps, tiles, s2s, dequant=True)
    torch.cuda.synchronize()
    for i in range(37):
        single = focus.quantize_mixfp4(ws[i], maps[i], tiles[i][0], tiles[i][1], s2s[i], dequant=True)
        torch.cuda.synchronize()
        assert torch.equal(b.outs[i].codes, single.codes) and torch.equal(b.outs[i].scales, single.scales)
        assert torch.equal(b.outs[i].deq.view(torch.int16), single.deq.view(torch.int16))
        c, sc, d = orc.mixfp4_quantize(np_bits(ws[i]), np.float32(s2s[i].item()), maps[i].cpu().numpy(),
                                       tiles[i][0], tiles[i][1])
        assert np.array_equal(single.codes.cpu().numpy(), c) and np.array_equal(single.scales.cpu().numpy(), sc)
        assert np.array_equal(np_bits(single.deq), d)


@pytest.mark.parametrize("shape,tile", MIX_CASES[:6], ids=lambda v: f"{v[0]}x{v[1]}")
def test_mixfp4_dequantize(focus, orc, shape, tile):
    """Stored MixFP4 back to BF16 against the oracle, and equal to the fused
    w' of the quantizer (the same map)."""
    rows, cols = shape
    w = synth.weights(shape, seed=rows + 5 * cols, tensor_id=26, zero_block_p=0.02)
    wb = np_bits(w)
    tmap = synth.tile_map(rows, cols, tile, frac=0.4, seed=rows, tensor_id=27).numpy()
    md = torch.from_numpy(tmap).to(DEV)
    res = focus.quantize_mixfp4(w.to(DEV), md, tile[0], tile[1], dequant=True)
    deq = focus.dequantize_mixfp4(res.codes, res.scales, res.s2, md, tile[0], tile[1])
    torch.cuda.synchronize()
    assert torch.equal(deq.view(torch.int16), res.deq.view(torch.int16))
    # the oracle on random stored bytes (every code and scale byte, both formats)
    rng = np.random.default_rng(rows)
    codes = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, (rows, cols // 16)).astype(np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x38  # no NaN scale bytes (NaN payloads are not compared)
    s2 = np.float32(3.0e-3)
    got = focus.dequantize_mixfp4(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                                  torch.tensor([s2], device=DEV), md, tile[0], tile[1])
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(got), orc.mixfp4_dequantize(codes, scales, s2, tmap, tile[0], tile[1]))
