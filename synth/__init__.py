"""Seeded synthetic inputs for the FOCUS NVFP4 quantizer.

This module serves both the oracle tests and the HIP path.  It draws random
numbers and lays out shapes; it holds none of the quantizer's arithmetic.

Shapes.  The weight sets are the quantized linear layers of Llama models (all
text-model linears except the LM head, "FOCUS NVFP4 scales for
Llama-3.2-1B-Instruct (our reproduction)", section "What this is"), written as
[out_features, in_features]:

* Llama-3.2-1B: 16 layers x {q 2048x2048, k 512x2048, v 512x2048,
  o 2048x2048, gate 8192x2048, up 8192x2048, down 2048x8192} = 112 linears;
* Llama-3.1-8B: 32 layers x {q 4096x4096, k/v 1024x4096, o 4096x4096,
  gate/up 14336x4096, down 4096x14336} = 224 linears;
* Llama-3.1-70B: 80 layers x {q/o 8192x8192, k/v 1024x8192,
  gate/up 28672x8192, down 8192x28672} = 560 linears.

Distributions (the checkpoints and calibration state are not available, so
these stand in for them): W ~ N(0, std) with a small fraction of entries
scaled up as outliers, rounded to BF16; m = 1 + U(-0.2, 0.2) or
LogNormal(0, 0.1) (the page initialises m at 1); q ~ N(6, 2) (initialised at
6); activations ~ N(0, 1) with a few outlier channels.

Random streams: every tensor has its own ``torch.Generator`` seeded with a
splitmix64 hash of (seed, tensor id), on the device the tensor is made on.
CPU and GPU generators give different bits for the same seed; parity never
relies on that, because the oracle always runs on the very bytes the GPU
consumed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import torch

MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, tensor_id: int) -> int:
    """63-bit seed of the random stream of one tensor."""
    return _splitmix64(_splitmix64(seed & MASK64) ^ (tensor_id & MASK64)) >> 1


def generator(seed: int, tensor_id: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, tensor_id))
    return g


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

def weights(shape: Tuple[int, int], *, seed: int, tensor_id: int, std: float = 0.02,
            outlier_p: float = 0.001, outlier_scale: float = 20.0,
            zero_block_p: float = 0.0, device="cpu") -> torch.Tensor:
    """BF16 weights [rows, cols]: N(0, std); each entry independently becomes
    an outlier (x outlier_scale, applied in FP32 before the BF16 rounding) with
    probability outlier_p; each 16-element block along a row is set to +0.0
    with probability zero_block_p."""
    rows, cols = shape
    g = generator(seed, tensor_id, device)
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    if outlier_p > 0:
        hit = torch.rand((rows, cols), generator=g, device=device) < outlier_p
        w = torch.where(hit, w * outlier_scale, w)
        del hit
    if zero_block_p > 0:
        assert cols % 16 == 0
        z = torch.rand((rows, cols // 16), generator=g, device=device) < zero_block_p
        w.view(rows, cols // 16, 16).masked_fill_(z.unsqueeze(-1), 0.0)
    return w.to(torch.bfloat16)


def block_factor_uniform(shape: Tuple[int, int], *, seed: int, tensor_id: int,
                         half_width: float = 0.2, device="cpu") -> torch.Tensor:
    """FP32 block factors m = 1 + U(-half_width, half_width)."""
    g = generator(seed, tensor_id, device)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return 1.0 + (2.0 * u - 1.0) * half_width


def block_factor_lognormal(shape: Tuple[int, int], *, seed: int, tensor_id: int,
                           sigma: float = 0.1, device="cpu") -> torch.Tensor:
    """FP32 block factors m ~ LogNormal(0, sigma)."""
    g = generator(seed, tensor_id, device)
    n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return torch.exp(n * sigma)


def logits(shape: Tuple[int, int], *, seed: int, tensor_id: int, mean: float = 6.0,
           std: float = 2.0, device="cpu") -> torch.Tensor:
    """FP32 sub-block logits q ~ N(mean, std)."""
    g = generator(seed, tensor_id, device)
    n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return n * std + mean


def activations(shape: Tuple[int, int], *, seed: int, tensor_id: int = 0,
                outlier_channel_p: float = 0.02, outlier_scale: float = 30.0,
                device="cpu") -> torch.Tensor:
    """BF16 activations [tokens, hidden] ~ N(0, 1); each hidden channel is an
    outlier channel (x outlier_scale) with probability outlier_channel_p."""
    t, h = shape
    g = generator(seed, tensor_id, device)
    x = torch.randn((t, h), generator=g, device=device, dtype=torch.float32)
    ch = torch.rand((h,), generator=g, device=device) < outlier_channel_p
    x = torch.where(ch.unsqueeze(0), x * outlier_scale, x)
    return x.to(torch.bfloat16)


def tile_map(rows: int, cols: int, tile: Tuple[int, int], *, frac: float, seed: int,
             tensor_id: int, device="cpu") -> torch.Tensor:
    """uint8 format map [rows/th, cols/tw], row-major: each tile is 1 (E0M3)
    independently with probability frac, else 0 (E2M1)."""
    th, tw = tile
    g = generator(seed, tensor_id, device)
    u = torch.rand((rows // th, cols // tw), generator=g, device=device)
    return (u < frac).to(torch.uint8)


def nvfp4_operand(rows: int, K: int, *, seed: int, tensor_id: int, scale_lo: int = 0x28,
                  scale_hi: int = 0x50, device="cpu"):
    """A stored NVFP4 tensor [rows, K] as random bytes: codes uniform over all
    256 byte values (two E2M1 codes each), scale bytes uniform over the
    normal E4M3 range [scale_lo, scale_hi)."""
    g = generator(seed, tensor_id, device)
    codes = torch.randint(0, 256, (rows, K // 2), generator=g, dtype=torch.uint8, device=device)
    scales = torch.randint(scale_lo, scale_hi, (rows, K // 16), generator=g, dtype=torch.uint8, device=device)
    return codes, scales


# E0M3 fraction of each published map: E0M3 tiles / all tiles.
MIXFP4_FRAC = {(8, 64): 83_771 / 13_631_488, (16, 64): 52_719 / 6_815_744, (256, 64): 9_447 / 425_984}


# ---------------------------------------------------------------------------
# weight sets
# ---------------------------------------------------------------------------

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class Linear:
    name: str
    layer: int
    proj: int
    rows: int
    cols: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    def tid(self, field: int) -> int:
        """Tensor id of field 0 (W), 1 (m), 2 (q), 3 (tile map) of this linear."""
        return (self.layer * 16 + self.proj) * 4 + field


@dataclass(frozen=True)
class WeightSet:
    name: str
    hidden: int
    kv: int
    inter: int
    layers: int
    std: float
    m_kind: str  # "uniform" or "lognormal"

    def linears(self) -> List[Linear]:
        h, kv, f = self.hidden, self.kv, self.inter
        shapes = [(h, h), (kv, h), (kv, h), (h, h), (f, h), (f, h), (h, f)]
        out = []
        for layer in range(self.layers):
            for p, (r, c) in enumerate(shapes):
                out.append(Linear(f"model.layers.{layer}.{PROJ[p]}", layer, p, r, c))
        return out

    def layer_shapes(self) -> List[Tuple[int, int]]:
        return [(l.rows, l.cols) for l in self.linears()[:7]]

    @property
    def numel(self) -> int:
        return sum(l.numel for l in self.linears())


LLAMA_1B = WeightSet("Llama-3.2-1B-shaped set (112 linears)", 2048, 512, 8192, 16, 0.02, "lognormal")
LLAMA_8B = WeightSet("Llama-3.1-8B-shaped set (224 linears)", 4096, 1024, 14336, 32, 0.02, "lognormal")
LLAMA_70B = WeightSet("Llama-3.1-70B-shaped set (560 linears)", 8192, 1024, 28672, 80, 0.015, "lognormal")

SINGLE_SHAPE = (256, 1024)
ACT_SHAPE = (8192, 4096)
SEED = 42


def make_linear(ws: WeightSet, lin: Linear, *, seed: int = SEED, device="cpu",
                with_m: bool = True, with_q: bool = True):
    """(W, m, q) of one linear of a weight set."""
    w = weights((lin.rows, lin.cols), seed=seed, tensor_id=lin.tid(0), std=ws.std,
                device=device)
    m = q = None
    if with_m:
        if ws.m_kind == "uniform":
            m = block_factor_uniform((lin.rows, lin.cols // 16), seed=seed,
                                     tensor_id=lin.tid(1), device=device)
        else:
            m = block_factor_lognormal((lin.rows, lin.cols // 16), seed=seed,
                                       tensor_id=lin.tid(1), device=device)
    if with_q:
        q = logits((lin.rows, lin.cols // 8), seed=seed, tensor_id=lin.tid(2), device=device)
    return w, m, q


def make_single(*, seed: int = SEED, device="cpu"):
    """The single-linear case [256, 1024]: N(0, 0.02), 0.1 % outliers x20,
    1 % of 16-blocks zeroed, m = 1 + U(-0.2, 0.2), q ~ N(6, 2)."""
    r, c = SINGLE_SHAPE
    w = weights((r, c), seed=seed, tensor_id=1, std=0.02, zero_block_p=0.01, device=device)
    m = block_factor_uniform((r, c // 16), seed=seed, tensor_id=2, device=device)
    q = logits((r, c // 8), seed=seed, tensor_id=3, device=device)
    return w, m, q


def make_activations(shape=ACT_SHAPE, *, seed: int = SEED, device="cpu"):
    """Per-token activation case: X [8192, 4096] ~ N(0, 1), 2 % of channels x30."""
    return activations(shape, seed=seed, tensor_id=7, device=device)


def bits(t: torch.Tensor):
    """numpy view of a tensor's raw bits (BF16 -> uint16), on the host."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
