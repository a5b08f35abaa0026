"""The synthetic weight sets reproduce the counts printed on the pages, and
the generators are deterministic (CPU only).  Sources in
tests/golden/page_counts.txt."""
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_counts.txt")


def page_counts():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v) if "." in v else int(v)
    return out


def test_llama_1b_counts_match_page():
    c = page_counts()
    lin = synth.LLAMA_1B.linears()
    assert len(lin) == c["linears_llama_3_2_1b"]
    assert sum(l.numel // 16 for l in lin) == c["m_total_llama_3_2_1b"]
    assert sum(l.numel // 8 for l in lin) == c["q_total_llama_3_2_1b"]
    assert synth.LLAMA_1B.numel == 973_078_528


def test_focus_state_size_means_fp32():
    """m and q of the 1B set in FP32 take (60,817,408 + 121,634,816) * 4 =
    729,808,896 bytes; focus.pt is 729,889,075 bytes, i.e. that plus ~80 kB of
    container, config and s2.  In FP16 it would be half as large."""
    c = page_counts()
    fp32 = (c["m_total_llama_3_2_1b"] + c["q_total_llama_3_2_1b"]) * 4
    assert 0 < c["focus_pt_bytes"] - fp32 < 100_000
    assert c["focus_pt_bytes"] > 1.9 * fp32 / 2


def test_llama_8b_tiles_match_page():
    """Every 8B linear is tiled exactly by 8x64, 16x64 and 256x64 tiles and
    the totals equal the page's tile counts."""
    c = page_counts()
    lin = synth.LLAMA_8B.linears()
    assert len(lin) == 224
    for (th, tw), key in [((8, 64), "tiles_8x64_llama_3_1_8b"), ((16, 64), "tiles_16x64_llama_3_1_8b"),
                          ((256, 64), "tiles_256x64_llama_3_1_8b")]:
        assert all(l.rows % th == 0 and l.cols % tw == 0 for l in lin)
        assert sum((l.rows // th) * (l.cols // tw) for l in lin) == c[key]
    assert synth.LLAMA_8B.numel == 6_979_321_856


def test_mixfp4_fractions_match_page():
    c = page_counts()
    for (th, tw), f in synth.MIXFP4_FRAC.items():
        key = f"{th}x{tw}_llama_3_1_8b"
        assert f == c["e0m3_tiles_" + key] / c["tiles_" + key]
    m = synth.tile_map(4096, 14336, (8, 64), frac=0.25, seed=1, tensor_id=3)
    assert m.shape == (512, 224) and m.dtype == torch.uint8
    assert abs(m.float().mean().item() - 0.25) < 0.01
    assert torch.equal(m, synth.tile_map(4096, 14336, (8, 64), frac=0.25, seed=1, tensor_id=3))


def test_llama_70b_count():
    assert len(synth.LLAMA_70B.linears()) == 560
    assert synth.LLAMA_70B.numel == 68_451_041_280


def test_storage_ratio():
    """NVFP4 stores 4 bits per element plus one 8-bit scale per 16: 4.5 bits,
    16 / 4.5 = 3.56x smaller than BF16, the ~3.5x the page reports."""
    c = page_counts()
    ratio = 16 / (4 + 8 / 16)
    assert abs(ratio - c["nvfp4_size_ratio_approx"]) < 0.1


def test_generators_deterministic_and_shaped():
    w1, m1, q1 = synth.make_single()
    w2, m2, q2 = synth.make_single()
    assert w1.dtype == torch.bfloat16 and w1.shape == (256, 1024)
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))
    assert torch.equal(m1, m2) and torch.equal(q1, q2)
    assert m1.shape == (256, 64) and q1.shape == (256, 128)
    assert float(m1.min()) >= 0.8 and float(m1.max()) <= 1.2
    zero_blocks = (w1.view(256, 64, 16).float().abs().amax(-1) == 0).sum().item()
    assert 100 < zero_blocks < 250  # 1 % of 16384 blocks
    x = synth.make_activations((64, 256))
    assert x.shape == (64, 256) and x.dtype == torch.bfloat16
    assert synth.stream_seed(42, 1) != synth.stream_seed(42, 2)
