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
* expf (the sigmoid's exponential, read as correctly rounded): every binary32
  argument in [-104, 89] (outside, the result is 0 or +inf), against binary64
  exp rounded once to binary32, which is the correctly rounded result unless
  the binary64 value lies within its own error of a binary32 midpoint; the
  arguments within 2^-40 (relative) of one are settled with decimal
  arithmetic at 60 digits.
"""
from decimal import Decimal, localcontext
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


def _f32_nearest(d):
    """The binary32 nearest to the Decimal d (d > 0, never a midpoint here:
    exp of a nonzero binary32 is irrational)."""
    f = np.float32(float(d))
    best = None
    for c in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Decimal(float(c)) - d)
        if best is None or err < best[0]:
            best = (err, c)
    return best[1]


def test_expf_every_binary32_in_range(orc):
    def check(bits):
        x = bits.view(np.float32)
        got = orc.expf_array(x)
        with np.errstate(over="ignore", under="ignore"):
            y = np.exp(x.astype(np.float64))
            f = y.astype(np.float32)
            toward = np.where(y > f.astype(np.float64), np.float32(np.inf), np.float32(-np.inf))
            mid = (f.astype(np.float64) + np.nextafter(f, toward).astype(np.float64)) * 0.5
        hard = np.abs(y - mid) <= np.abs(y) * 2.0 ** -40
        bad = int(np.count_nonzero((got.view(np.uint32) != f.view(np.uint32)) & ~hard))
        with localcontext() as ctx:
            ctx.prec = 60
            for xi, gi in zip(x[hard], got[hard]):
                want = _f32_nearest(Decimal(float(xi)).exp())
                bad += int(np.float32(gi).view(np.uint32) != want.view(np.uint32))
        return bad

    neg_hi = np.float32(-104.0).view(np.uint32).item() + 1
    pos_hi = np.float32(89.0).view(np.uint32).item() + 1
    assert _sweep(0x80000000, neg_hi, check) == 0  # -0 .. -104
    assert _sweep(0, pos_hi, check) == 0           # +0 .. 89
    edge = np.array([-200.0, -104.5, 89.5, 1e30, np.inf, -np.inf], dtype=np.float32)
    assert np.array_equal(orc.expf_array(edge), np.array([0, 0, np.inf, np.inf, np.inf, 0], dtype=np.float32))

