"""The library under HIP graph capture: every call is asynchronous on the
caller's stream, allocates nothing and records no memset, so a decode-like
sequence (tensor scale, quantize with w', per-token activations, the linear
layer with and without a k split) can be captured once and replayed.  Each
replay, with eager work and synchronizations between replays, must give the
eager results bit for bit."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def focus():
    import fp4_post_weight_amd as f
    f._lib.lib()
    assert torch.cuda.is_available()
    return f


def _sequence(focus, w, m, q, x, wl_codes, wl_scales, wl_s2, outs):
    """One pass; writes into the preallocated ``outs`` (graph-stable addresses)."""
    focus.tensor_scale(w, s2_out=outs["s2"], amax_out=outs["amax"])
    focus.quantize(w, m, q, outs["s2"], dequant=True, out=outs["wq"])
    focus.quantize_act_per_token(x, out=outs["xq"])
    wl = focus.Quantized(wl_codes, wl_scales, None, wl_s2)
    # N = 1024, K = 28672 splits k (partials in the workspace, then the
    # finalize kernel); N = 4096, K = 4096 does not
    focus.nvfp4_linear(outs["xq"], wl, out_dtype=torch.float32, out=outs["y_split"], workspace=outs["ws"])
    w2 = focus.Quantized(outs["wq"].codes, outs["wq"].scales, None, outs["s2"])
    x2 = focus.Quantized(outs["xq2"].codes, outs["xq2"].scales, None, outs["xq2"].s2)
    focus.nvfp4_linear(x2, w2, out_dtype=torch.bfloat16, out=outs["y"], workspace=None)


def test_graph_replays_match_eager(focus):
    torch.manual_seed(0)
    rows, cols, tokens = 4096, 4096, 16
    w = (torch.randn((rows, cols), device=DEV) * 0.02).to(torch.bfloat16)
    m = 1.0 + 0.2 * (torch.rand((rows, cols // 16), device=DEV) - 0.5)
    q = 6.0 + 2.0 * torch.randn((rows, cols // 8), device=DEV)
    x = torch.randn((tokens, 28672), device=DEV).to(torch.bfloat16)
    x2 = torch.randn((tokens, cols), device=DEV).to(torch.bfloat16)
    wl_codes, wl_scales = synth.nvfp4_operand(1024, 28672, seed=5, tensor_id=1, device=DEV)
    wl_s2 = torch.tensor([2.0e-3], device=DEV)
    ws_bytes = focus.nvfp4_linear_workspace_bytes(tokens, 1024, 28672)
    assert ws_bytes > 0
    outs = {
        "s2": torch.empty(1, dtype=torch.float32, device=DEV),
        "amax": torch.empty(1, dtype=torch.float32, device=DEV),
        "wq": focus.Quantized(torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV),
                              torch.empty((rows, cols // 16), dtype=torch.uint8, device=DEV),
                              torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV), None),
        "xq": focus.Quantized(torch.empty((tokens, 28672 // 2), dtype=torch.uint8, device=DEV),
                              torch.empty((tokens, 28672 // 16), dtype=torch.uint8, device=DEV), None,
                              torch.empty(tokens, dtype=torch.float32, device=DEV)),
        "y_split": torch.empty((tokens, 1024), dtype=torch.float32, device=DEV),
        "y": torch.empty((tokens, rows), dtype=torch.bfloat16, device=DEV),
        "ws": torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV),
    }
    outs["xq2"] = focus.quantize_act_per_token(x2)
    names = ("s2", "amax", "y_split", "y")

    def snapshot():
        torch.cuda.synchronize()
        snap = {k: outs[k].clone() for k in names}
        snap.update(wq_codes=outs["wq"].codes.clone(), wq_scales=outs["wq"].scales.clone(),
                    wq_deq=outs["wq"].deq.clone(), xq_codes=outs["xq"].codes.clone(),
                    xq_scales=outs["xq"].scales.clone(), xq_s2=outs["xq"].s2.clone())
        return snap

    _sequence(focus, w, m, q, x, wl_codes, wl_scales, wl_s2, outs)
    eager = snapshot()

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up on the capture stream
        _sequence(focus, w, m, q, x, wl_codes, wl_scales, wl_s2, outs)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _sequence(focus, w, m, q, x, wl_codes, wl_scales, wl_s2, outs)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: overwrite every output with garbage
        for k in names:
            outs[k].fill_(float("nan") if outs[k].is_floating_point() else 7)
        outs["wq"].codes.fill_(0x55)
        outs["wq"].deq.fill_(1.0)
        outs["xq"].codes.fill_(0x33)
        outs["ws"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for k, v in eager.items():
            a, b = v.view(torch.uint8) if v.dtype != torch.uint8 else v, got[k]
            b = b.view(torch.uint8) if b.dtype != torch.uint8 else b
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager result"


def test_batched_graph_replays_match_eager(focus):
    """The batched calls of a weight-set step (tensor scale, quantize with w',
    dequantize) and the batched FourOverSix and MixFP4 quantizers, prepared
    once, captured together and replayed: every replay gives the eager bytes."""
    shapes = [(256, 4096), (1024, 1024), (48, 1536), (8, 64), (200, 14336)]
    ws = [(torch.randn(s, device=DEV) * (0.01 * (i + 1))).to(torch.bfloat16) for i, s in enumerate(shapes)]
    ms = [1.0 + 0.2 * (torch.rand((r, c // 16), device=DEV) - 0.5) for r, c in shapes]
    qs = [6.0 + 2.0 * torch.randn((r, c // 8), device=DEV) for r, c in shapes]
    maps = [synth.tile_map(r, c, (8, 64), frac=0.3, seed=9, tensor_id=i, device=DEV)
            for i, (r, c) in enumerate(shapes)]
    n = len(shapes)
    s2 = torch.empty((n, 1), dtype=torch.float32, device=DEV)
    amax = torch.empty((n, 1), dtype=torch.float32, device=DEV)
    s2s = [s2[i] for i in range(n)]

    def outs():
        return [focus.Quantized(torch.empty((r, c // 2), dtype=torch.uint8, device=DEV),
                                torch.empty((r, c // 16), dtype=torch.uint8, device=DEV),
                                torch.empty((r, c), dtype=torch.bfloat16, device=DEV), s2s[i])
                for i, (r, c) in enumerate(shapes)]

    oq, of, om = outs(), outs(), outs()
    deq = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    batches = [
        focus.tensor_scale_many(ws, s2, amax, run=False),
        focus.quantize_many(ws, ms, qs, s2s, outs=oq, dequant=True, run=False),
        focus.dequantize_many([o.codes for o in oq], [o.scales for o in oq], s2s, outs=deq, run=False),
        focus.quantize_fo6_many(ws, s2s, outs=of, dequant=True, run=False),
        focus.quantize_mixfp4_many(ws, maps, [(8, 64)] * n, s2s, outs=om, dequant=True, run=False),
    ]
    bufs = [s2, amax] + deq + [t for o in oq + of + om for t in (o.codes, o.scales, o.deq)]

    def step():
        for b in batches:
            b.run()

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in bufs]

    step()
    eager = snapshot()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in bufs:  # eager work between replays
            t.fill_(float("nan") if t.is_floating_point() else 0x5A)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for k, (a, b) in enumerate(zip(eager, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: buffer {k} differs"
