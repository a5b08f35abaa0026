"""The Python binding rejects caller-supplied output buffers of the wrong
dtype, device or size before anything is launched: each case fills the
buffers with a sentinel, expects the exception, then checks after a device
synchronization that no byte of any buffer changed.  Runs on an MI355X only
(marker gpu)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def focus():
    import fp4_post_weight_amd as f
    f._lib.lib()
    return f


def _sentinel(*ts):
    for t in ts:
        if t is not None:
            t.view(torch.uint8).fill_(0xA5) if t.dtype != torch.uint8 else t.fill_(0xA5)
    return [None if t is None else t.clone() for t in ts]


def _unchanged(ts, saved):
    torch.cuda.synchronize()
    for t, s in zip(ts, saved):
        if t is not None:
            assert torch.equal(t.view(torch.uint8), s.view(torch.uint8))


def _w(rows=64, cols=256):
    g = torch.Generator(device="cpu").manual_seed(rows * 7 + cols)
    return (torch.randn(rows, cols, generator=g) * 0.02).to(torch.bfloat16).to(DEV)


def _bufs(rows, cols, scale_block=16, s2_rows=0, short=None):
    b = {"codes": torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV),
         "scales": torch.empty((rows, cols // scale_block), dtype=torch.uint8, device=DEV),
         "deq": torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV),
         "s2": torch.empty((max(s2_rows, 1),), dtype=torch.float32, device=DEV)}
    if short is not None:  # one row too few
        t = b[short]
        b[short] = t.view(-1)[: t.numel() - max(1, t.numel() // max(rows, 1))]
    return b


@pytest.mark.parametrize("short", ["codes", "scales", "deq"])
def test_quantize_out_too_small(focus, short):
    w = _w()
    s2, _ = focus.tensor_scale(w)
    b = _bufs(64, 256, short=short)
    ts = [b["codes"], b["scales"], b["deq"]]
    saved = _sentinel(*ts)
    with pytest.raises(ValueError):
        focus.quantize(w, s2=s2, dequant=True, out=focus.Quantized(b["codes"], b["scales"], b["deq"], s2))
    _unchanged(ts, saved)


def test_quantize_out_wrong_dtype_and_device(focus):
    w = _w()
    s2, _ = focus.tensor_scale(w)
    b = _bufs(64, 256)
    with pytest.raises(TypeError):
        focus.quantize(w, s2=s2, out=focus.Quantized(b["codes"].view(torch.int8), b["scales"], b["deq"], s2))
    with pytest.raises(ValueError):
        focus.quantize(w, s2=s2, out=focus.Quantized(b["codes"].cpu(), b["scales"], b["deq"], s2))
    with pytest.raises(ValueError):  # dequant requested, no w' buffer given
        focus.quantize(w, s2=s2, dequant=True, out=focus.Quantized(b["codes"], b["scales"], None, s2))


@pytest.mark.parametrize("fo6", [False, True], ids=["nvfp4", "fo6"])
@pytest.mark.parametrize("short", ["codes", "scales", "s2", "deq"])
def test_act_per_token_out_too_small(focus, fo6, short):
    x = _w(48, 512)
    b = _bufs(48, 512, s2_rows=48, short=short)
    ts = [b["codes"], b["scales"], b["s2"], b["deq"]]
    saved = _sentinel(*ts)
    call = focus.quantize_act_per_token_fo6 if fo6 else focus.quantize_act_per_token
    with pytest.raises(ValueError):
        call(x, dequant=True, out=focus.Quantized(b["codes"], b["scales"], b["deq"], b["s2"]))
    _unchanged(ts, saved)


@pytest.mark.parametrize("short", ["codes", "scales", "deq"])
def test_fo6_out_too_small(focus, short):
    w = _w()
    s2, _ = focus.tensor_scale(w)
    b = _bufs(64, 256, short=short)
    ts = [b["codes"], b["scales"], b["deq"]]
    saved = _sentinel(*ts)
    with pytest.raises(ValueError):
        focus.quantize_fo6(w, s2, dequant=True, out=focus.Quantized(b["codes"], b["scales"], b["deq"], s2))
    _unchanged(ts, saved)


def test_dequantize_out_too_small(focus):
    w = _w()
    r = focus.quantize(w, dequant=False)
    out = torch.empty(64 * 256 - 16, dtype=torch.bfloat16, device=DEV)
    saved = _sentinel(out)
    with pytest.raises(ValueError):
        focus.dequantize(r.codes, r.scales, r.s2, out=out)
    with pytest.raises(ValueError):
        focus.dequantize_mx(r.codes, r.scales.view(-1)[: 64 * 8].view(64, 8), out=out)
    _unchanged([out], saved)


def test_many_calls_check_every_buffer(focus):
    ws = [_w(32, 256), _w(16, 512)]
    s2 = torch.empty((2, 1), dtype=torch.float32, device=DEV)
    focus.tensor_scale_many(ws, s2)
    good = [_bufs(32, 256), _bufs(16, 512)]
    bad = _bufs(16, 512, short="deq")
    outs = [focus.Quantized(good[0]["codes"], good[0]["scales"], good[0]["deq"], s2[0]),
            focus.Quantized(bad["codes"], bad["scales"], bad["deq"], s2[1])]
    ts = [good[0]["codes"], good[0]["scales"], good[0]["deq"], bad["codes"], bad["scales"], bad["deq"]]
    saved = _sentinel(*ts)
    with pytest.raises(ValueError):
        focus.quantize_many(ws, [None, None], [None, None], [s2[0], s2[1]], outs=outs, dequant=True)
    with pytest.raises(ValueError):  # m of the wrong shape (no longer an assert)
        focus.quantize_many(ws, [torch.ones((32, 8), device=DEV), None], [None, None], [s2[0], s2[1]])
    with pytest.raises(ValueError):
        focus.dequantize_many([good[0]["codes"], bad["codes"]], [good[0]["scales"], bad["scales"]],
                              [s2[0], s2[1]], outs=[good[0]["deq"], bad["deq"]])
    with pytest.raises(ValueError):
        focus.quantize_mx_many(ws, [torch.ones((32, 4), device=DEV), None], [None, None])
    _unchanged(ts, saved)
