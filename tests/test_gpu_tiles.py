"""Launch-tile boundaries.  Each streaming kernel takes 256 lanes x (blocks
per lane) 16-element blocks per tile: NVFP4 with w' 512, without 768,
FourOverSix without w' 1280, with w' 512, MXFP4 with w' 256, without 512,
MixFP4 with w' 768, the dequantize 256; a batched call lays its tensors'
tiles end to end.  One batched call per path over tensors one block short
of, at and one past those boundaries (and past two tiles), every output
against the oracle.  Runs on an MI355X only (marker gpu)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# blocks per tensor: around 256, 512, 768 and 1280
NBLK = [1, 255, 256, 257, 511, 512, 513, 767, 768, 769, 1279, 1280, 1281, 2561]


@pytest.fixture(scope="module")
def focus():
    import fp4_post_weight_amd as f
    return f


def _bits(t):
    return synth.bits(t)


def _weights(nblk_list, seed, cols_mult=16):
    """One row per tensor, nblk 16-element blocks (cols_mult 32: an even
    count for 32-element blocks)."""
    ws = []
    for i, n in enumerate(nblk_list):
        cols = cols_mult * n
        ws.append(synth.weights((1, cols), seed=seed + i, tensor_id=40, zero_block_p=0.02).to(DEV))
    return ws


@pytest.mark.parametrize("dequant", [True, False])
def test_nvfp4_tiles(focus, orc, dequant):
    ws = _weights(NBLK, 500)
    ms = [synth.block_factor_lognormal((1, w.shape[1] // 16), seed=600 + i, tensor_id=41).to(DEV)
          for i, w in enumerate(ws)]
    qs = [synth.logits((1, w.shape[1] // 8), seed=700 + i, tensor_id=42).to(DEV) for i, w in enumerate(ws)]
    ts = focus.tensor_scale_many(ws)
    b = focus.quantize_many(ws, ms, qs, [ts.s2[i] for i in range(len(ws))], dequant=dequant)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        s2 = np.float32(ts.s2[i].item())
        c, sc, d = orc.quantize(_bits(w.cpu()), ms[i].cpu().numpy(), qs[i].cpu().numpy(), s2, dequant=dequant)
        assert np.array_equal(b.outs[i].scales.cpu().numpy(), sc), NBLK[i]
        assert np.array_equal(b.outs[i].codes.cpu().numpy(), c), NBLK[i]
        if dequant:
            assert np.array_equal(_bits(b.outs[i].deq), d), NBLK[i]


@pytest.mark.parametrize("dequant", [True, False])
def test_fo6_tiles(focus, orc, dequant):
    ws = _weights(NBLK, 800)
    ts = focus.tensor_scale_many(ws)
    b = focus.quantize_fo6_many(ws, [ts.s2[i] for i in range(len(ws))], dequant=dequant)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        c, sc, d = orc.fo6_quantize(_bits(w.cpu()), np.float32(ts.s2[i].item()), dequant=dequant)
        assert np.array_equal(b.outs[i].scales.cpu().numpy(), sc), NBLK[i]
        assert np.array_equal(b.outs[i].codes.cpu().numpy(), c), NBLK[i]
        if dequant:
            assert np.array_equal(_bits(b.outs[i].deq), d), NBLK[i]


@pytest.mark.parametrize("dequant", [True, False])
def test_mx_tiles(focus, orc, dequant):
    # 32-element blocks: twice the 16-element block counts above, halved
    nb32 = [max(1, n // 2) for n in NBLK] + [128, 129, 256, 257]
    ws = _weights(nb32, 900, cols_mult=32)
    ms = [synth.block_factor_lognormal((1, w.shape[1] // 32), seed=1000 + i, tensor_id=43).to(DEV)
          for i, w in enumerate(ws)]
    qs = [synth.logits((1, w.shape[1] // 8), seed=1100 + i, tensor_id=44).to(DEV) for i, w in enumerate(ws)]
    b = focus.quantize_mx_many(ws, ms, qs, dequant=dequant)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        c, sc, d = orc.mx_quantize(_bits(w.cpu()), ms[i].cpu().numpy(), qs[i].cpu().numpy(), dequant=True)
        assert np.array_equal(b.outs[i].scales.cpu().numpy(), sc), nb32[i]
        assert np.array_equal(b.outs[i].codes.cpu().numpy(), c), nb32[i]
        if dequant:
            assert np.array_equal(_bits(b.outs[i].deq), d), nb32[i]


def test_mixfp4_tiles(focus, orc):
    ws = _weights(NBLK, 1200)
    maps = [synth.tile_map(1, w.shape[1], (1, 16), frac=0.3, seed=1300 + i, tensor_id=45, device=DEV)
            for i, w in enumerate(ws)]
    ts = focus.tensor_scale_many(ws)
    s2s = [ts.s2[i] for i in range(len(ws))]
    b = focus.quantize_mixfp4_many(ws, maps, [(1, 16)] * len(ws), s2s, dequant=True)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        c, sc, d = orc.mixfp4_quantize(_bits(w.cpu()), np.float32(s2s[i].item()), maps[i].cpu().numpy(), 1, 16)
        assert np.array_equal(b.outs[i].scales.cpu().numpy(), sc), NBLK[i]
        assert np.array_equal(b.outs[i].codes.cpu().numpy(), c), NBLK[i]
        assert np.array_equal(_bits(b.outs[i].deq), d), NBLK[i]


def test_dequantize_tiles(focus, orc):
    ws = _weights(NBLK, 1400)
    ts = focus.tensor_scale_many(ws)
    s2s = [ts.s2[i] for i in range(len(ws))]
    q = focus.quantize_fo6_many(ws, s2s, dequant=False)
    dq = focus.dequantize_many([o.codes for o in q.outs], [o.scales for o in q.outs], s2s)
    torch.cuda.synchronize()
    for i in range(len(ws)):
        want = orc.dequantize(q.outs[i].codes.cpu().numpy(), q.outs[i].scales.cpu().numpy(),
                              np.float32(s2s[i].item()))
        assert np.array_equal(_bits(dq.outs[i]), want), NBLK[i]


def test_mixed_runs_in_one_batch(focus, orc):
    """A batched call whose entries alternate between codes only and codes
    + w' is split into runs of one kernel each, and the two kernels use
    different tile sizes (FourOverSix 1280 and 512 blocks, MXFP4 512 and
    256): every entry against the oracle."""
    ws = _weights(NBLK, 1500)
    ts = focus.tensor_scale_many(ws)
    s2s = [ts.s2[i] for i in range(len(ws))]
    outs = [focus.Quantized(torch.empty((1, w.shape[1] // 2), dtype=torch.uint8, device=DEV),
                            torch.empty((1, w.shape[1] // 16), dtype=torch.uint8, device=DEV),
                            torch.empty((1, w.shape[1]), dtype=torch.bfloat16, device=DEV) if i % 2 else None,
                            s2s[i]) for i, w in enumerate(ws)]
    b = focus.quantize_fo6_many(ws, s2s, outs=outs, dequant=True)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        c, sc, d = orc.fo6_quantize(_bits(w.cpu()), np.float32(s2s[i].item()), dequant=True)
        assert np.array_equal(b.outs[i].scales.cpu().numpy(), sc), NBLK[i]
        assert np.array_equal(b.outs[i].codes.cpu().numpy(), c), NBLK[i]
        if i % 2:
            assert np.array_equal(_bits(b.outs[i].deq), d), NBLK[i]
        else:
            assert b.outs[i].deq is None
    nb32 = [max(1, n // 2) for n in NBLK]
    wm = _weights(nb32, 1600, cols_mult=32)
    om = [focus.Quantized(torch.empty((1, w.shape[1] // 2), dtype=torch.uint8, device=DEV),
                          torch.empty((1, w.shape[1] // 32), dtype=torch.uint8, device=DEV),
                          torch.empty((1, w.shape[1]), dtype=torch.bfloat16, device=DEV) if i % 2 else None,
                          None) for i, w in enumerate(wm)]
    bm = focus.quantize_mx_many(wm, [None] * len(wm), [None] * len(wm), outs=om, dequant=True)
    torch.cuda.synchronize()
    for i, w in enumerate(wm):
        c, sc, d = orc.mx_quantize(_bits(w.cpu()), None, None, dequant=True)
        assert np.array_equal(bm.outs[i].scales.cpu().numpy(), sc), nb32[i]
        assert np.array_equal(bm.outs[i].codes.cpu().numpy(), c), nb32[i]
        if i % 2:
            assert np.array_equal(_bits(bm.outs[i].deq), d), nb32[i]
