"""Exhaustive sweeps of the oracle's three format roundings (CPU only,
marked slow): every binary32 input of the range each one is used on, against
an independent formulation.

* E2M1 (equation c_i's rounding, ties to the even code): every non-NaN
  binary32 of either sign against the decision-interval table (the tie at
  each boundary going to the code with mantissa bit 0, saturation beyond 6).
* E4M3 (equation S_b's rounding): every binary32 t in [2^-6, 448], the range
  the clamp leaves, against torch's float8_e4m3fn conversion.
* BF16 (equation w'_i's rounding): every finite binary32 against torch's
  bfloat16 conversion.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.slow

CHUNK = 1 << 24


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _sweep(lo, hi, fn):
    """fn(bits uint32 array) -> number of mismatches, over [lo, hi)."""
    starts = list(range(lo, hi, CHUNK))
    with ThreadPoolExecutor(_threads()) as ex:
        bad = list(ex.map(lambda s: fn(np.arange(s, min(s + CHUNK, hi), dtype=np.uint32)), starts))
    return sum(bad)


def e2m1_by_intervals(x):
    a = np.abs(x)
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) +
           (a > 5.0))
    return mag | ((x.view(np.uint32) >> 31).astype(np.uint8) << 3)


def test_e2m1_every_binary32(orc):
    def check(bits):
        out = 0
        for sign in (0, 0x80000000):
            x = (bits | np.uint32(sign)).view(np.float32)
            out += int(np.count_nonzero(orc.e2m1_round_array(x) != e2m1_by_intervals(x)))
        return out
    assert _sweep(0, 0x7F800001, check) == 0  # +0 .. +inf and -0 .. -inf


def test_e4m3_every_clamped_binary32(orc):
    lo = np.float32(2.0 ** -6).view(np.uint32).item()
    hi = np.float32(448.0).view(np.uint32).item() + 1

    def check(bits):
        t = bits.view(np.float32)
        ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return int(np.count_nonzero(orc.e4m3_round_array(t) != ref))
    assert _sweep(lo, hi, check) == 0


def test_bf16_every_finite_binary32(orc):
    def check(bits):
        out = 0
        for sign in (0, 0x80000000):
            x = (bits | np.uint32(sign)).view(np.float32)
            ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            out += int(np.count_nonzero(orc.bf16_round_array(x) != ref))
        return out
    assert _sweep(0, 0x7F800000, check) == 0  # every finite magnitude, both signs
