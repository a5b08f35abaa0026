"""The quantizer's device arithmetic helpers, checked on the GPU (marker gpu).

Two kinds of check, through the test-only library tests/hip (built from the
same numerics header as the product kernels):
  * exhaustive sweeps over binary32 inputs against an independent device
    formulation of the same rule (IEEE division, integer RNE, the E2M1
    definition, the platform exp): these back the exactness arguments stated
    in fp4_post_weight_amd/csrc/focus_numerics.h;
  * structured and random inputs compared with the CPU oracle.
"""
import ctypes as ct
import os
import struct

import numpy as np
import pytest
import torch

import oracle_pins as pins

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libfocus_selftest.so")
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def st():
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libfocus_selftest.so is not built (run __graft_entry__.build())")
    lib = ct.CDLL(LIB)
    lib.focus_selftest_exhaustive.argtypes = [ct.c_int, ct.POINTER(ct.c_ulonglong)]
    lib.focus_selftest_exhaustive.restype = ct.c_int
    lib.focus_selftest_map.argtypes = [ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int64]
    lib.focus_selftest_map.restype = ct.c_int
    return lib


def exhaustive(st, which):
    r = ct.c_ulonglong(0)
    assert st.focus_selftest_exhaustive(which, ct.byref(r)) == 0
    return r.value


def dmap(st, which, x, out_dtype, x2=None):
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    x2d = None if x2 is None else torch.from_numpy(np.ascontiguousarray(x2)).to(DEV)
    out = torch.empty(xd.numel(), dtype=out_dtype, device=DEV)
    assert st.focus_selftest_map(which, xd.data_ptr(), 0 if x2d is None else x2d.data_ptr(),
                                 out.data_ptr(), xd.numel()) == 0
    return out.cpu().numpy()


# ---- exhaustive --------------------------------------------------------------

def test_corrected_reciprocal_is_ieee_below_2_126(st):
    """1/s of the sigmoid: every binary32 s in [1, 2^126)."""
    assert exhaustive(st, 0) == 0


def test_binary64_reciprocal_error(st):
    """recip_f64: |r*d - 1| <= 2^-52.5 for every positive binary32 d (the
    element-quotient argument needs well below 2^-50)."""
    worst = struct.unpack("<d", struct.pack("<Q", exhaustive(st, 1)))[0]
    print(f"largest relative residual 2^{np.log2(worst):.2f}")
    assert worst <= 2.0 ** -52.5


def test_exp_matches_platform_exp_everywhere(st):
    """exp_f64 rounded to binary32 equals the platform binary64 exp rounded to
    binary32 for every binary32 in [-105, 89]."""
    assert exhaustive(st, 2) == 0


def test_hardware_e2m1_packing_exhaustive(st):
    """v_cvt_scalef32_pk_fp4_f32 (scale 1) = clamp + nearest-even E2M1 with
    signed zeros, for every non-NaN binary32, all eight nibble slots."""
    assert exhaustive(st, 3) == 0


def test_hardware_bf16_exhaustive(st):
    """v_cvt_pk_bf16_f32 = round to nearest even for every non-NaN binary32."""
    assert exhaustive(st, 4) == 0


# ---- against the oracle --------------------------------------------------------

def _near(center_bits, k):
    return (np.arange(-k, k + 1, dtype=np.int64) + center_bits).astype(np.uint32)


def test_e2m1_against_oracle(st, orc):
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    near = np.concatenate([_near(int(b), 2000) for b in bounds.view(np.uint32)]).view(np.float32)
    rng = np.random.default_rng(41)
    rand = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, -3.4e38, 6.0001, 100.0], np.float32)
    x = np.concatenate([near, -near, rand, special]).astype(np.float32)
    x = x[~np.isnan(x)]
    if x.size % 2:
        x = x[:-1]
    got = dmap(st, 0, x, torch.uint8)
    want = orc.e2m1_round_array(np.clip(x, np.float32(-6), np.float32(6)))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]).hex(), int(got[i]), int(want[i])) for i in bad[:8]]


def test_bf16_against_oracle(st, orc):
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    if x.size % 2:
        x = x[:-1]
    got = dmap(st, 1, x, torch.int16).view(np.uint16)
    want = orc.bf16_round_array(x)
    assert np.array_equal(got, want)


def test_e4m3_against_oracle(st, orc):
    t = pins.e4m3_probe_values()
    got = dmap(st, 4, t, torch.uint8)
    assert np.array_equal(got, orc.e4m3_round_array(t))


def test_expf_and_sigmoid_against_oracle(st, orc):
    rng = np.random.default_rng(42)
    q = np.concatenate([
        np.linspace(-100, 100, 1_000_001, dtype=np.float32),
        (rng.standard_normal(2_000_000) * 2 + 6).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 16.0, 17.0, 24 * np.log(2), -87.0, -88.0, -88.8, -89.0,
                  -103.0, 104.0, 1e-30, -1e-30], np.float32)])
    e_dev = dmap(st, 3, -q, torch.float32)
    e_orc = orc.expf_array(-q)
    assert np.array_equal(e_dev.view(np.uint32), e_orc.view(np.uint32))
    s_dev = dmap(st, 2, q, torch.float32)
    s_orc = orc.sigmoid_array(q)
    assert np.array_equal(s_dev.view(np.uint32), s_orc.view(np.uint32))


def test_quotients_are_ieee(st):
    """The element quotient RN32(RN64(w * recip_f64(d))) and the block quotient
    RN32(RN64(num * RN64(1/den))) equal IEEE binary32 division (numpy) on
    random BF16 w / binary32 d of every exponent, and on random binary32 pairs."""
    rng = np.random.default_rng(43)
    n = 4_000_000
    w = pins.bf16_float(rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16))
    d = rng.integers(1, 0x7F7FFFFF, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    ok = np.isfinite(w)
    w, d = w[ok], d[ok]
    with np.errstate(all="ignore"):
        want = (w / d).astype(np.float32)
    got = dmap(st, 5, w, torch.float32, x2=d)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    num = rng.integers(0, 0x7F7FFFFF, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    den = rng.integers(1, 0x7F7FFFFF, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    with np.errstate(all="ignore"):
        want = (num / den).astype(np.float32)
    got = dmap(st, 6, num, torch.float32, x2=den)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
