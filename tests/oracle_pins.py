"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Every ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with the pin.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle
with planted mistakes and requires each mistake to be caught.

Sources of the pins (page titles and sections):
  P1 "FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our reproduction)",
     section "What this is": field table (m, q, s2), equations S_b, c_i,
     w'_i and the paragraph after them (ties to even, zero-block rule,
     plain NVFP4 storage), activations with one scale per token.
  Library routines: torch's float8_e4m3fn and bfloat16 conversions (IEEE /
  OCP round-to-nearest-even), Python's math.exp (binary64).
  Closed forms derived from the equations, stated at each check.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

E2M1_VALUES = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


# ---------------------------------------------------------------------------
# independent helpers (library routines, no oracle code)
# ---------------------------------------------------------------------------

def torch_bf16_bits(x) -> np.ndarray:
    """float32 -> BF16 bits with torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_float(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def torch_e4m3_bytes(t) -> np.ndarray:
    x = torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_value(b) -> np.ndarray:
    x = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return x.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] codes, element 2j = low nibble."""
    lo = packed & 0xF
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)


def code_value(codes) -> np.ndarray:
    codes = np.asarray(codes)
    v = E2M1_VALUES[codes & 7]
    return np.where(codes & 8, -v, v)


def read_golden_e2m1():
    xs, cs = [], []
    with open(os.path.join(GOLDEN, "e2m1_intervals.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            x, c = line.split()
            xs.append(float.fromhex(x) if "inf" not in x else float(x))
            cs.append(int(c, 16))
    return np.array(xs, dtype=np.float32), np.array(cs, dtype=np.uint8)


def ulp32(x: float) -> float:
    x = abs(np.float32(x))
    return float(np.spacing(x))


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def check_e2m1_table(o):
    """Hand-written interval table (tests/golden/e2m1_intervals.txt): every
    decision boundary, one ulp either side, the values, saturation, signed
    zeros.  The clamp to [-6, 6] of equation c_i is applied first."""
    xs, cs = read_golden_e2m1()
    got = o.e2m1_round_array(np.clip(xs, -6, 6))
    bad = np.nonzero(got != cs)[0]
    assert bad.size == 0, [(float(xs[i]).hex(), int(cs[i]), int(got[i])) for i in bad[:8]]


def check_e2m1_nearest_dense(o):
    """Every float with its 13 low mantissa bits clear in [-6, 6] (about
    1.3 M values, both signs) rounds to a nearest E2M1 value: no other value
    is closer.  Brute force over the 8 magnitudes."""
    pos = np.arange(0, 0x40C00001, 1 << 13, dtype=np.uint32).view(np.float32)
    xs = np.concatenate([pos, -pos]).astype(np.float32)
    got = o.e2m1_round_array(xs)
    dist_got = np.abs(np.abs(xs.astype(np.float64)) - E2M1_VALUES[got & 7])
    dist_all = np.abs(np.abs(xs.astype(np.float64))[:, None] - E2M1_VALUES[None, :])
    assert np.all(dist_got <= dist_all.min(axis=1))
    assert np.all(((got >> 3) & 1) == np.signbit(xs))


def e4m3_probe_values():
    """Structured binary32 values in [2^-6, 448]: all 2^11 settings of
    mantissa bits 12..22 with the low 12 bits 0x000 / 0x001 / 0xFFF (covers
    every tie and near tie of a 3-bit rounding), exponents -6..8."""
    base = np.arange(0x3C800000, 0x43E00001, 1 << 12, dtype=np.uint64)
    vals = np.concatenate([base, base + 1, base + 0xFFF])
    vals = vals[(vals >= 0x3C800000) & (vals <= 0x43E00000)].astype(np.uint32)
    return vals.view(np.float32)


def check_e4m3_vs_torch(o):
    """E4M3 round-to-nearest-even of equation S_b agrees with torch's
    float8_e4m3fn conversion on every tie-relevant value of [2^-6, 448]."""
    t = e4m3_probe_values()
    got = o.e4m3_round_array(t)
    want = torch_e4m3_bytes(t)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(t[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def check_e4m3_decode_vs_torch(o):
    """E4M3 decoding agrees with torch for all 254 finite bytes."""
    bs = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    want = torch_e4m3_value(bs)
    got = np.array([o.e4m3_value(int(b)) for b in bs], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def check_bf16_vs_torch(o):
    """BF16 round-to-nearest-even (w' of equation w'_i) agrees with torch on
    every upper half with lower halves 0x0000/0x0001/0x7FFF/0x8000/0x8001/
    0xFFFF (every tie and near tie) plus 200k random finite values."""
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(5)
    u = np.concatenate([u, rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = o.bf16_round_array(x)
    want = torch_bf16_bits(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x[i].view(np.uint32))), hex(int(got[i])), hex(int(want[i])))
                           for i in bad[:8]]


# ---------------------------------------------------------------------------
# sigmoid and exp
# ---------------------------------------------------------------------------

def check_sigmoid(o):
    """sigmoid(q) = 1/(1+exp(-q)): closed forms and binary64 math.exp.

    sigmoid(0) = 1/2 exactly; sigmoid(+inf) = 1; for q >= 17, exp(-q) is
    below half an ulp of 1 so 1 + e rounds to 1 and sigmoid is exactly 1;
    sigmoid(6) (the page's initial q) is 0.99752737684336523...; every value
    is within 2 binary32 ulps of the binary64 formula."""
    assert o.sigmoid(0.0) == 0.5
    assert o.sigmoid(float("inf")) == 1.0
    assert o.sigmoid(17.0) == 1.0 and o.sigmoid(40.0) == 1.0
    assert o.sigmoid(16.0) < 1.0
    s6 = 1.0 / (1.0 + math.exp(-6.0))
    assert abs(o.sigmoid(6.0) - s6) <= ulp32(s6)
    qs = np.linspace(-20, 20, 4001, dtype=np.float32)
    got = o.sigmoid_array(qs).astype(np.float64)
    want = np.array([1.0 / (1.0 + math.exp(-float(q))) for q in qs])
    tol = 2 * np.spacing(want.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= tol)


def check_expf_correctly_rounded(o):
    """expf is read as the correctly rounded binary32 exponential: it must
    equal binary64 math.exp rounded once to binary32 (which is the correct
    rounding except within 2^-29 of a midpoint) on 20k random arguments."""
    rng = np.random.default_rng(7)
    xs = rng.uniform(-87, 88, 20_000).astype(np.float32)
    got = np.array([o.expf(float(x)) for x in xs], dtype=np.float32)
    want = np.array([math.exp(float(x)) for x in xs], dtype=np.float64).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# tensor scale
# ---------------------------------------------------------------------------

def check_tensor_scale(o):
    """s2 = amax|W| / (6*448) (field table, row s2): closed forms."""
    w = torch_bf16_bits(np.array([2688.0, -1.0, 0.5, 0.0], np.float32))
    s2, amax = o.tensor_scale(w)
    assert s2 == np.float32(1.0) and amax == np.float32(2688.0)
    w = torch_bf16_bits(np.array([3.0, -5376.0], np.float32))
    s2, amax = o.tensor_scale(w)
    assert s2 == np.float32(2.0) and amax == np.float32(5376.0)
    s2, amax = o.tensor_scale(np.zeros(0, np.uint16))
    assert s2 == 0 and amax == 0
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(10_000) * 0.02).astype(np.float32)
    wb = torch_bf16_bits(x)
    s2, amax = o.tensor_scale(wb)
    ref = np.max(np.abs(bf16_float(wb)))
    assert amax == ref
    assert s2 == np.float32(ref) / np.float32(2688.0)


# ---------------------------------------------------------------------------
# the quantizer: fixed points built from the equations
# ---------------------------------------------------------------------------

S2_POW2 = np.float32(2.0 ** -10)


def _fixed_point_case(rng, n_rows=119, nb=4):
    """Rows r = 0..118 use the E4M3 scale byte 0x08 + r (every normal
    value).  Each 16-block holds w_i = c_i * S * s2 with random codes c_i and
    one |c| = 6; all such w_i are exact in BF16 (at most 6 significant
    bits), so with m = 1 and sigmoid = 1 equation S_b gives t = S exactly,
    and c_i = w_i / (S * s2) exactly."""
    sbytes = (0x08 + np.arange(n_rows)).astype(np.uint8)
    S = torch_e4m3_value(sbytes).astype(np.float64)
    codes = rng.integers(0, 16, (n_rows, nb * 16)).astype(np.uint8)
    pos = rng.integers(0, 16, (n_rows, nb))
    for r in range(n_rows):
        for b in range(nb):
            codes[r, 16 * b + pos[r, b]] = 7 | (codes[r, 16 * b + pos[r, b]] & 8)
    w = code_value(codes) * S[:, None] * float(S2_POW2)
    wb = torch_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_float(wb).astype(np.float64), w), "construction not exact"
    # signed zeros: code 8 must come from -0.0
    wb = np.where(codes == 8, np.uint16(0x8000), wb).astype(np.uint16)
    return sbytes, S, codes, wb


def check_fixed_points(o):
    """P1 equations S_b, c_i, w'_i at their fixed points: the quantizer
    returns the scale byte and codes the block was built from, packs element
    2j into the low nibble, and w' = w bit for bit."""
    rng = np.random.default_rng(11)
    sbytes, S, codes, wb = _fixed_point_case(rng)
    pc, sc, wd = o.quantize(wb, None, None, S2_POW2)
    assert np.all(sc == sbytes[:, None])
    assert np.array_equal(unpack_codes(pc), codes)
    assert np.array_equal(wd, wb)
    # q = +inf (sigmoid exactly 1) and q = 20 give the same result
    q = np.full((wb.shape[0], wb.shape[1] // 8), np.inf, np.float32)
    pc2, sc2, wd2 = o.quantize(wb, np.ones((wb.shape[0], wb.shape[1] // 16), np.float32), q, S2_POW2)
    assert np.array_equal(pc2, pc) and np.array_equal(sc2, sc) and np.array_equal(wd2, wd)
    q[:] = 20.0
    pc3, _, _ = o.quantize(wb, None, q, S2_POW2)
    assert np.array_equal(pc3, pc)


# E2M1 of c/2, by hand from the interval table: magnitude code k -> code of
# half its value (0.25 and 0.75 are ties that go to the even code).
HALF_MAP = np.array([0, 0, 1, 2, 2, 3, 4, 5], dtype=np.uint8)
# E2M1 of clamp(2c, -6, 6): 0->0, 0.5->1, 1->2, 1.5->3, 2->4, 3->6, 4->8->6, 6->12->6
DOUBLE_MAP = np.array([0, 2, 4, 5, 6, 7, 7, 7], dtype=np.uint8)


def check_block_factor_m(o):
    """Equation S_b with m_b in {1, 2} chosen per block (rows 0..110, so
    2S <= 448): t = S * m_b, so the scale byte is that of 2S where m_b = 2,
    and the codes are E2M1(c/2) there (interval table, ties to even).  A
    transposed or shifted index of m fails this."""
    rng = np.random.default_rng(12)
    sbytes, S, codes, wb = _fixed_point_case(rng, n_rows=111, nb=5)
    m2 = rng.integers(0, 2, (111, 5)).astype(bool)
    m = np.where(m2, np.float32(2.0), np.float32(1.0)).astype(np.float32)
    pc, sc, wd = o.quantize(wb, m, None, S2_POW2)
    want_sc = np.where(m2, torch_e4m3_bytes((2 * S[:, None]).astype(np.float32) * np.ones((1, 5), np.float32)),
                       sbytes[:, None])
    assert np.array_equal(sc, want_sc)
    want_c = codes.copy()
    mask16 = np.repeat(m2, 16, axis=1)
    halved = (codes & 8) | HALF_MAP[codes & 7]
    want_c[mask16] = halved[mask16]
    assert np.array_equal(unpack_codes(pc), want_c)
    Sb = torch_e4m3_value(sc).astype(np.float64)
    want_w = code_value(want_c) * np.repeat(Sb, 16, axis=1) * float(S2_POW2)
    want_wb = torch_bf16_bits(want_w.astype(np.float32))
    want_wb = np.where(want_c == 8, np.uint16(0x8000), want_wb)
    assert np.array_equal(wd, want_wb)


def check_subblock_logits(o):
    """Equation c_i with sigmoid(q_k): q = 0 gives sigmoid exactly 1/2, so
    that sub-block's codes become E2M1(clamp(2c)); q = +inf leaves them.
    Sub-blocks are chosen at random per (row, block, k): a swapped k or a
    transposed q index fails this.  The scale bytes do not depend on q."""
    rng = np.random.default_rng(13)
    sbytes, S, codes, wb = _fixed_point_case(rng, n_rows=119, nb=3)
    half = rng.integers(0, 2, (119, 6)).astype(bool)
    q = np.where(half, np.float32(0.0), np.float32(np.inf)).astype(np.float32)
    pc, sc, wd = o.quantize(wb, None, q, S2_POW2)
    assert np.all(sc == sbytes[:, None])
    mask8 = np.repeat(half, 8, axis=1)
    doubled = (codes & 8) | DOUBLE_MAP[codes & 7]
    want_c = np.where(mask8, doubled, codes)
    assert np.array_equal(unpack_codes(pc), want_c)


def check_zero_blocks(o):
    """Zero-block rule (paragraph after the equations): a block whose scaled
    maximum is 0 takes scale 1 (byte 0x38), codes of +0 are 0x0, of -0 are
    0x8 (sign-preserving reading), w' keeps the signed zero.  m_b = 0 makes
    the scaled maximum 0 as well."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    wb = torch_bf16_bits(x)
    wb[0, 16:32] = 0x0000
    wb[1, 0:16] = 0x8000
    wb[2, 48:64] = np.array([0x0000, 0x8000] * 8, np.uint16)
    m = np.ones((4, 4), np.float32)
    m[3, 2] = 0.0
    s2, _ = o.tensor_scale(wb)
    pc, sc, wd = o.quantize(wb, m, None, s2)
    assert sc[0, 1] == 0x38 and sc[1, 0] == 0x38 and sc[2, 3] == 0x38 and sc[3, 2] == 0x38
    c = unpack_codes(pc)
    assert np.all(c[0, 16:32] == 0) and np.all(wd[0, 16:32] == 0)
    assert np.all(c[1, 0:16] == 8) and np.all(wd[1, 0:16] == 0x8000)
    assert np.array_equal(c[2, 48:64], np.array([0, 8] * 8))
    assert np.array_equal(wd[2, 48:64], np.array([0, 0x8000] * 8))


def check_clamps(o):
    """The clamp of equation S_b to [2^-6, 448]: with s2 = 1 (amax 2688), a
    block of maximum 0.01 has t = 0.01/6 < 2^-6 and takes byte 0x08 (2^-6,
    the smallest normal E4M3; subnormal scales never arise); the amax block
    with m_b = 10 has t = 4480 > 448 and takes byte 0x7E, its maximum element
    then has x = 2688 / 448 = 6 (code 7)."""
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 1:16] = 1.0
    x[1, 16] = -0.01
    x[1, 17:32] = 0.001
    wb = torch_bf16_bits(x)
    s2, _ = o.tensor_scale(wb)
    assert s2 == 1.0
    m = np.ones((2, 2), np.float32)
    m[0, 0] = 10.0
    pc, sc, _ = o.quantize(wb, m, None, s2)
    assert sc[1, 1] == 0x08 and sc[0, 0] == 0x7E
    c = unpack_codes(pc)
    assert c[0, 0] == 7
    # S = 2^-6: x = -0.01 * 64 = -0.64 -> -0.5 (code 9)
    assert c[1, 16] == 9


def check_s2_zero(o):
    """s2 = 0 (an all-zero tensor; the page leaves 0/0 undefined): every
    block is a zero block, scale byte 0x38, signed-zero codes and w'."""
    wb = np.zeros((3, 32), np.uint16)
    wb[1, 5] = 0x8000
    s2, amax = o.tensor_scale(wb)
    assert s2 == 0 and amax == 0
    pc, sc, wd = o.quantize(wb, None, None, s2)
    assert np.all(sc == 0x38)
    c = unpack_codes(pc)
    assert c[1, 5] == 8 and np.count_nonzero(c) == 1
    assert np.array_equal(wd, wb)


# ---------------------------------------------------------------------------
# the quantizer on random data: closed forms, bounds, invariants
# ---------------------------------------------------------------------------

def _random_case(seed, rows=96, cols=512, with_q=True, m_none=True):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    out = rng.random((rows, cols)) < 0.002
    x[out] *= 20
    wb = torch_bf16_bits(x)
    m = None if m_none else np.exp(0.1 * rng.standard_normal((rows, cols // 16))).astype(np.float32)
    q = (rng.standard_normal((rows, cols // 8)) * 2 + 6).astype(np.float32) if with_q else None
    return wb, m, q


def check_amax_block_closed_form(o):
    """With m = 1, the block holding amax|W| has t = amax / (6 * (amax/2688))
    = 448 * (1 +- 2^-22), which clamps and rounds to 448: scale byte 0x7E.
    Its maximum element then has |x| >= 6 / (1 + 2^-4) > 5 for any sigmoid
    <= 1, so its code magnitude is 6 (code 7)."""
    for seed in range(4):
        wb, _, q = _random_case(100 + seed)
        s2, amax = o.tensor_scale(wb)
        pc, sc, _ = o.quantize(wb, None, q, s2)
        mag = np.abs(bf16_float(wb))
        r, col = np.unravel_index(np.argmax(mag), mag.shape)
        assert sc[r, col // 16] == 0x7E
        c = unpack_codes(pc)
        assert (c[r, col] & 7) == 7
        # every block: its own maximum element maps to magnitude >= 4 when
        # sigmoid = 1 and the block scale is not clamped (S >= t/(1+2^-4))
    wb, _, _ = _random_case(200)
    s2, _ = o.tensor_scale(wb)
    pc, sc, _ = o.quantize(wb, None, None, s2)
    c = unpack_codes(pc).reshape(wb.shape[0], -1, 16)
    mag = np.abs(bf16_float(wb)).reshape(wb.shape[0], -1, 16)
    S = torch_e4m3_value(sc)
    amax_b = mag.max(axis=2)
    t = amax_b / (6 * s2)
    unclamped = (t > 2 ** -6) & (t < 448)
    top = np.take_along_axis(c, mag.argmax(axis=2)[..., None], axis=2)[..., 0] & 7
    assert np.all(top[unclamped] >= 6)
    assert np.all(S > 0)


GAP = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])  # larger spacing next to |c|


def check_error_bound(o):
    """Equation w'_i with sigmoid = 1: an element that is not clamped lies
    within half an E2M1 step of its code, scaled by S*s2, plus the BF16
    rounding of w' (half a BF16 ulp) and the binary32 roundings (2^-22
    relative)."""
    wb, m, _ = _random_case(300, m_none=False)
    s2, _ = o.tensor_scale(wb)
    pc, sc, wd = o.quantize(wb, m, None, s2)
    w = bf16_float(wb).astype(np.float64)
    wp = bf16_float(wd).astype(np.float64)
    c = unpack_codes(pc)
    S = np.repeat(torch_e4m3_value(sc).astype(np.float64), 16, axis=1)
    x = w / (S * float(s2))
    inside = np.abs(x) <= 6.0
    # one BF16 ulp is 2^16 binary32 ulps (7 instead of 23 mantissa bits)
    ulp_bf16 = np.spacing(np.abs(wp).astype(np.float32)).astype(np.float64) * 65536.0
    bound = 0.5 * GAP[c & 7] * S * float(s2) + 0.5 * ulp_bf16 + 2.0 ** -22 * np.abs(wp)
    err = np.abs(w - wp)
    assert np.all(err[inside] <= bound[inside])
    assert np.all(np.abs(code_value(c)) <= 6)


def check_monotone(o):
    """Within a sub-block the denominator is positive, so sorting by w gives
    non-decreasing code values."""
    wb, m, q = _random_case(400, m_none=False)
    s2, _ = o.tensor_scale(wb)
    pc, _, _ = o.quantize(wb, m, q, s2)
    v = code_value(unpack_codes(pc)).reshape(-1, 8)
    w = bf16_float(wb).astype(np.float64).reshape(-1, 8)
    order = np.argsort(w, axis=1, kind="stable")
    vs = np.take_along_axis(v, order, axis=1)
    assert np.all(np.diff(vs, axis=1) >= 0)


def plain_nvfp4_rtn(wb: np.ndarray, s2: np.float32):
    """Textbook NVFP4 round-to-nearest (the page's "NVFP4" baseline row):
    block scale from torch's E4M3 conversion, codes from the E2M1 decision
    boundaries (x > 0.25, >= 0.75, > 1.25, >= 1.75, > 2.5, >= 3.5, > 5).
    Written independently of the oracle, in vectorised binary32 numpy."""
    rows, cols = wb.shape
    w = bf16_float(wb).reshape(rows, cols // 16, 16)
    a = np.abs(w).max(axis=2).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (a / (np.float32(6.0) * s2)).astype(np.float32)
    t = np.where(t == 0, np.float32(1.0), t)
    t = np.clip(t, np.float32(2 ** -6), np.float32(448)).astype(np.float32)
    sb = torch_e4m3_bytes(t)
    S = torch_e4m3_value(sb)
    d = (S * s2).astype(np.float32)
    x = (w / d[..., None]).astype(np.float32)
    x = np.clip(x, np.float32(-6), np.float32(6))
    ax = np.abs(x)
    mag = ((ax > 0.25).astype(np.uint8) + (ax >= 0.75) + (ax > 1.25) + (ax >= 1.75)
           + (ax > 2.5) + (ax >= 3.5) + (ax > 5)).astype(np.uint8)
    code = (np.signbit(x).astype(np.uint8) << 3) | mag
    return code.reshape(rows, cols), sb


def check_plain_rtn_reduction(o):
    """m = 1 with no relaxation (q = None or q = +inf) is plain NVFP4
    round-to-nearest: scale bytes and codes equal the textbook quantizer."""
    for seed in (500, 501):
        wb, _, _ = _random_case(seed)
        s2, _ = o.tensor_scale(wb)
        pc, sc, _ = o.quantize(wb, None, None, s2)
        codes, sb = plain_nvfp4_rtn(wb, s2)
        assert np.array_equal(sc, sb)
        assert np.array_equal(unpack_codes(pc), codes)


def check_dequantize_roundtrip(o):
    """Dequantizing the stored codes and scales gives the fused w'
    (equation w'_i computed from the stored NVFP4 data)."""
    wb, m, q = _random_case(600, m_none=False)
    s2, _ = o.tensor_scale(wb)
    pc, sc, wd = o.quantize(wb, m, q, s2)
    assert np.array_equal(o.dequantize(pc, sc, s2), wd)
    s2r = np.full(wb.shape[0], s2, np.float32)
    assert np.array_equal(o.dequantize(pc, sc, s2r, s2_per_row=True), wd)


def check_act_per_token(o):
    """One scale per token: row t has s2_t = amax|x_t| / 2688, and each row's
    maximum block has scale byte 0x7E (closed form above with m = 1)."""
    rng = np.random.default_rng(700)
    x = rng.standard_normal((24, 256)).astype(np.float32)
    ch = rng.random(256) < 0.05
    x[:, ch] *= 30
    x[5] = 0.0
    xb = torch_bf16_bits(x)
    pc, sc, s2, xd = o.quantize_act_per_token(xb, dequant=True)
    amax = np.abs(bf16_float(xb)).max(axis=1)
    assert np.array_equal(s2, (amax / np.float32(2688.0)).astype(np.float32))
    mag = np.abs(bf16_float(xb))
    for t in range(24):
        if t == 5:
            assert np.all(sc[t] == 0x38) and np.all(pc[t] == 0)
            continue
        assert sc[t, int(np.argmax(mag[t])) // 16] == 0x7E
    # rows agree with the weight quantizer run on that row with m = 1, no q
    for t in (0, 7, 23):
        c1, s1, d1 = o.quantize(xb[t:t + 1], None, None, s2[t])
        assert np.array_equal(c1[0], pc[t]) and np.array_equal(s1[0], sc[t])
        assert np.array_equal(d1[0], xd[t])


# ---------------------------------------------------------------------------
# FourOverSix
# ---------------------------------------------------------------------------

def _fo6_four_case(rng, n_blocks=300):
    """Blocks w = c * S * s2 with S a power of two in [2^-6, 2^8], codes of
    magnitude <= 4 and one element of magnitude exactly 4.  The 4-candidate
    has t = a/(4*s2) = S exactly, so it reproduces the block with zero error;
    the 6-candidate's scale is E4M3(2S/3), which for a power of two S is not
    2S/3 (no E4M3 value is), so its maximum element is off: FourOverSix must
    choose the 4-candidate and return (S, c)."""
    exps = rng.integers(-6, 9, n_blocks)
    S = np.exp2(exps).astype(np.float64)
    mags = rng.integers(0, 7, (n_blocks, 16))          # codes 0..6 (values <= 4)
    signs = rng.integers(0, 2, (n_blocks, 16)) << 3
    pos = rng.integers(0, 16, n_blocks)
    mags[np.arange(n_blocks), pos] = 6                 # value 4
    codes = (mags | signs).astype(np.uint8)
    w = code_value(codes) * S[:, None] * float(S2_POW2)
    wb = torch_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_float(wb).astype(np.float64), w)
    wb = np.where(codes == 8, np.uint16(0x8000), wb).astype(np.uint16)
    sbytes = torch_e4m3_bytes(S.astype(np.float32))
    return sbytes, codes, wb.reshape(n_blocks // 4, 64), codes.reshape(n_blocks // 4, 64)


def check_fo6_four_fixed_points(o):
    rng = np.random.default_rng(60)
    sbytes, _, wb, codes = _fo6_four_case(rng)
    pc, sc, wd = o.fo6_quantize(wb, S2_POW2)
    assert np.array_equal(sc.ravel(), sbytes)
    assert np.array_equal(unpack_codes(pc), codes)
    assert np.array_equal(wd, wb)


def check_fo6_six_fixed_points(o):
    """Blocks with |c| = 6 at the maximum reproduce exactly under the
    6-candidate (error 0), so FourOverSix keeps it."""
    rng = np.random.default_rng(61)
    sbytes, S, codes, wb = _fixed_point_case(rng, n_rows=119, nb=3)
    pc, sc, wd = o.fo6_quantize(wb, S2_POW2)
    assert np.all(sc == sbytes[:, None])
    assert np.array_equal(unpack_codes(pc), codes)
    assert np.array_equal(wd, wb)


def check_fo6_ties_keep_six(o):
    """Ties: codes from {0, +-1.5, +-3, +-6} with one +-6 and S = 2^k
    (k = -6..8) are reproduced exactly by both candidates (the 4-candidate's
    scale 1.5*S is an E4M3 value and c/1.5 is an E2M1 value), so both errors
    are 0 and the 6-candidate, scale byte of S with codes c, must be kept."""
    rng = np.random.default_rng(64)
    n = 300
    S = np.exp2(rng.integers(-6, 9, n)).astype(np.float64)
    mags = np.array([0, 3, 5, 7], np.uint8)[rng.integers(0, 4, (n, 16))]
    mags[np.arange(n), rng.integers(0, 16, n)] = 7
    codes = (mags | (rng.integers(0, 2, (n, 16)) << 3)).astype(np.uint8)
    w = code_value(codes) * S[:, None] * float(S2_POW2)
    wb = torch_bf16_bits(w.astype(np.float32))
    wb = np.where(codes == 8, np.uint16(0x8000), wb).astype(np.uint16).reshape(n // 4, 64)
    pc, sc, wd = o.fo6_quantize(wb, S2_POW2)
    assert np.array_equal(sc.ravel(), torch_e4m3_bytes(S.astype(np.float32)))
    assert np.array_equal(unpack_codes(pc), codes.reshape(n // 4, 64))


def check_fo6_never_worse_than_rtn(o):
    """Per block, FourOverSix's squared error is at most plain NVFP4
    round-to-nearest's (it takes the 4-candidate only when that is lower),
    and the amax block keeps byte 0x7E (t = 672 clamps to 448 = the
    6-candidate's scale, a tie)."""
    wb, _, _ = _random_case(62)
    s2, _ = o.tensor_scale(wb)
    pc, sc, wd = o.fo6_quantize(wb, s2)
    pr, sr, wr = o.quantize(wb, None, None, s2)
    w = bf16_float(wb).astype(np.float64).reshape(-1, 16)
    def block_err(pcodes, sbytes):
        v = code_value(unpack_codes(pcodes)).reshape(-1, 16) * \
            torch_e4m3_value(sbytes).astype(np.float64).reshape(-1, 1) * float(s2)
        return ((w - v) ** 2).sum(axis=1)
    e_fo6, e_rtn = block_err(pc, sc), block_err(pr, sr)
    assert np.all(e_fo6 <= e_rtn * (1 + 1e-5) + 1e-30)
    changed = sc.ravel() != sr.ravel()
    assert changed.any() and np.all(e_fo6[changed] < e_rtn[changed] * (1 + 1e-5))
    mag = np.abs(bf16_float(wb))
    r, col = np.unravel_index(np.argmax(mag), mag.shape)
    assert sc[r, col // 16] == 0x7E


def check_fo6_zero_and_act(o):
    """Zero blocks and an all-zero token take byte 0x38; each token equals the
    per-tensor FourOverSix of that row with s2_t = amax|x_t| / 2688."""
    rng = np.random.default_rng(63)
    x = rng.standard_normal((12, 128)).astype(np.float32)
    x[:, rng.random(128) < 0.05] *= 30
    x[3] = 0.0
    x[5, 16:32] = 0.0
    xb = torch_bf16_bits(x)
    pc, sc, s2, xd = o.fo6_quantize_act_per_token(xb, dequant=True)
    assert np.all(sc[3] == 0x38) and sc[5, 1] == 0x38
    amax = np.abs(bf16_float(xb)).max(axis=1)
    assert np.array_equal(s2, (amax / np.float32(2688.0)).astype(np.float32))
    for t in (0, 5, 11):
        c1, s1, d1 = o.fo6_quantize(xb[t:t + 1], s2[t])
        assert np.array_equal(c1[0], pc[t]) and np.array_equal(s1[0], sc[t]) and np.array_equal(d1[0], xd[t])


# ---------------------------------------------------------------------------
# FOCUS on MXFP4
# ---------------------------------------------------------------------------

def unpack_mx_scales(sb):
    return np.exp2(sb.astype(np.float64) - 127.0)


def check_mx_scale_closed_forms(o):
    """OCP Microscaling block scale 2^(floor(log2 t) - 2): maxima 6*2^k and
    4*2^k and 7.99*2^k give 2^k (byte 127 + k), 3.99*2^k gives 2^(k-1); zero
    gives 1; the exponent clamps to [-127, 127]."""
    for k in range(-100, 101, 7):
        for mult, off in ((6.0, 0), (4.0, 0), (7.99, 0), (3.99, -1), (1.0, -2), (0.5, -3)):
            t = np.float32(mult * 2.0 ** k)
            assert o.mx_block_scale(t) == 127 + k + off, (mult, k)
    assert o.mx_block_scale(0.0) == 127
    assert o.mx_block_scale(2.0 ** -140) == 0
    assert o.mx_block_scale(1.5 * 2.0 ** 127) == 127 + 125
    assert o.mx_block_scale(3.0, 2.0) == 127 + 0  # t = a * m = 6
    for b in range(0, 255):
        assert o.e8m0_value(b) == np.float32(2.0 ** (b - 127))


def _mx_fixed_case(rng, rows=40, nb=4):
    """Blocks of 32 built as c * 2^k with one |c| in {4, 6}: floor(log2 max)
    = k + 2, so the scale is 2^k and the codes are c, exactly."""
    k = rng.integers(-100, 101, (rows, nb))
    codes = rng.integers(0, 16, (rows, nb * 32)).astype(np.uint8)
    pos = rng.integers(0, 32, (rows, nb))
    top = rng.choice(np.array([6, 7], np.uint8), (rows, nb))
    for r in range(rows):
        for b in range(nb):
            i = 32 * b + pos[r, b]
            codes[r, i] = (codes[r, i] & 8) | top[r, b]
    S = np.repeat(np.exp2(k.astype(np.float64)), 32, axis=1)
    w = code_value(codes) * S
    wb = torch_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_float(wb).astype(np.float64), w)
    wb = np.where(codes == 8, np.uint16(0x8000), wb).astype(np.uint16)
    return (k + 127).astype(np.uint8), codes, wb


def check_mx_fixed_points(o):
    rng = np.random.default_rng(80)
    sb, codes, wb = _mx_fixed_case(rng)
    pc, sc, wd = o.mx_quantize(wb, None, None)
    assert np.array_equal(sc, sb)
    assert np.array_equal(unpack_codes(pc), codes)
    assert np.array_equal(wd, wb)


def check_mx_factor_and_subblocks(o):
    """m_b = 2 doubles the scale (byte + 1) and halves the codes (E2M1(c/2),
    ties to even); q = 0 (sigmoid 1/2) doubles the codes of exactly that
    8-element sub-block, k = 0..3, through q[r, 4b + k]."""
    rng = np.random.default_rng(81)
    sb, codes, wb = _mx_fixed_case(rng, rows=24, nb=5)
    m2 = rng.integers(0, 2, (24, 5)).astype(bool)
    m = np.where(m2, 2.0, 1.0).astype(np.float32)
    pc, sc, _ = o.mx_quantize(wb, m, None, dequant=False)
    assert np.array_equal(sc, np.where(m2, sb + 1, sb))
    want = codes.copy()
    mask = np.repeat(m2, 32, axis=1)
    want[mask] = ((codes & 8) | HALF_MAP[codes & 7])[mask]
    assert np.array_equal(unpack_codes(pc), want)
    half = rng.integers(0, 2, (24, 20)).astype(bool)
    q = np.where(half, np.float32(0.0), np.float32(np.inf)).astype(np.float32)
    pc, sc, _ = o.mx_quantize(wb, None, q, dequant=False)
    assert np.array_equal(sc, sb)
    mask8 = np.repeat(half, 8, axis=1)
    want = np.where(mask8, (codes & 8) | DOUBLE_MAP[codes & 7], codes)
    assert np.array_equal(unpack_codes(pc), want)


def check_mx_plain_reduction(o):
    """m = 1 with no relaxation is plain OCP MXFP4 round-to-nearest, written
    independently here: shared exponent floor(log2 amax) - 2 from numpy's
    frexp, elements scaled by an exact power of two, E2M1 by its decision
    boundaries; dequantize(codes, scales) equals the fused w'."""
    wb, _, _ = _random_case(82, rows=64, cols=512)
    wb[3, 32:64] = 0
    pc, sc, wd = o.mx_quantize(wb, None, None)
    w = bf16_float(wb).astype(np.float32).reshape(64, 16, 32)
    a = np.abs(w).max(axis=2)
    _, e2 = np.frexp(a)
    e = np.where(a == 0, 0, np.clip(e2 - 1 - 2, -127, 127))
    x = np.clip(w * np.exp2(-e.astype(np.float64))[..., None], -6, 6).astype(np.float32)
    ax = np.abs(x)
    mag = ((ax > 0.25).astype(np.uint8) + (ax >= 0.75) + (ax > 1.25) + (ax >= 1.75)
           + (ax > 2.5) + (ax >= 3.5) + (ax > 5)).astype(np.uint8)
    want = ((np.signbit(x).astype(np.uint8) << 3) | mag).reshape(64, 512)
    assert np.array_equal(sc, (e + 127).astype(np.uint8))
    assert np.array_equal(unpack_codes(pc), want)
    assert np.array_equal(o.mx_dequantize(pc, sc), wd)
    assert np.all(sc[3, 1] == 127) and np.all(unpack_codes(pc)[3, 32:64] == 0)


# ---------------------------------------------------------------------------
# FlipQuant MixFP4
# ---------------------------------------------------------------------------

def check_e0m3_levels(o):
    """E0M3 = uniform levels 0..7 (FlipQuant page, "What this is"): nearest
    integer, ties to the even one, sign kept, after the clamp to [-7, 7]."""
    table = [(0.0, 0), (0.5, 0), (np.nextafter(np.float32(0.5), 1), 1), (1.5, 2), (2.5, 2),
             (3.5, 4), (4.5, 4), (5.5, 6), (6.5, 6), (np.nextafter(np.float32(6.5), 7), 7), (7.0, 7),
             (-0.0, 8), (-0.3, 8), (-7.0, 15), (-2.5, 10), (3.49, 3)]
    for x, code in table:
        assert o.e0m3_round(float(np.float32(x))) == code, (x, code)
    assert [o.e0m3_value(c) for c in (0, 7, 8, 13)] == [0.0, 7.0, -0.0, -5.0]


def _e0m3_fixed_case(rng, rows=24, nb=8):
    """Blocks c * S * s2 with integer levels c (|c| <= 7, one |c| = 7) and every
    normal E4M3 scale: t = 7*S*s2 / (7*s2) = S exactly."""
    sb = rng.integers(0x08, 0x7F, (rows, nb)).astype(np.uint8)
    S = torch_e4m3_value(sb).astype(np.float64)
    codes = rng.integers(0, 16, (rows, nb * 16)).astype(np.uint8)
    pos = rng.integers(0, 16, (rows, nb))
    for r in range(rows):
        for b in range(nb):
            codes[r, 16 * b + pos[r, b]] |= 7
    lv = (codes & 7).astype(np.float64) * np.where(codes & 8, -1.0, 1.0)
    w = lv * np.repeat(S, 16, axis=1) * float(S2_POW2)
    wb = torch_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_float(wb).astype(np.float64), w)
    wb = np.where(codes == 8, np.uint16(0x8000), wb).astype(np.uint16)
    return sb, codes, wb


def check_mixfp4_maps(o):
    """All-clear map = FourOverSix everywhere; all-set map = E0M3 everywhere,
    whose fixed points return (S, levels) and w' = w; a random 8x64 map on a
    16 x 256 tensor selects per tile exactly (a transposed or shifted tile
    index fails)."""
    rng = np.random.default_rng(95)
    sb, codes, wb = _e0m3_fixed_case(rng, rows=16, nb=16)
    ones = np.ones((2, 4), np.uint8)
    pc, sc, wd = o.mixfp4_quantize(wb, S2_POW2, ones, 8, 64)
    assert np.array_equal(sc, sb) and np.array_equal(unpack_codes(pc), codes) and np.array_equal(wd, wb)
    wr, _, _ = _random_case(96, rows=16, cols=256)
    s2, _ = o.tensor_scale(wr)
    z = o.mixfp4_quantize(wr, s2, np.zeros((2, 4), np.uint8), 8, 64)
    f = o.fo6_quantize(wr, s2)
    assert all(np.array_equal(a, b) for a, b in zip(z, f))
    e = o.mixfp4_quantize(wr, s2, ones, 8, 64)
    tmap = np.array([[1, 1, 0, 0], [0, 0, 1, 0]], np.uint8)
    mx = o.mixfp4_quantize(wr, s2, tmap, 8, 64)
    sel_blocks = np.repeat(np.repeat(tmap, 8, axis=0), 4, axis=1).astype(bool)   # [16, 16] blocks
    assert np.array_equal(mx[1], np.where(sel_blocks, e[1], f[1]))
    sel_el = np.repeat(sel_blocks, 16, axis=1)
    assert np.array_equal(unpack_codes(mx[0]), np.where(sel_el, unpack_codes(e[0]), unpack_codes(f[0])))
    assert np.array_equal(mx[2], np.where(sel_el, e[2], f[2]))


def check_mixfp4_dequantize(o):
    """Dequantizing stored MixFP4 gives the quantizer's fused w' bit for bit
    (random data, a mixed map), and hand-written E0M3 codes read as levels:
    codes 0x7 / 0xF / 0x8 with scale 1 and s2 = 2^-10 are +7, -7, -0 times
    2^-10, the same bytes in an E2M1 tile +6, -6, -0."""
    w, _, _ = _random_case(97, rows=32, cols=384)
    s2, _ = o.tensor_scale(w)
    tmap = np.array([[1, 0, 1, 0, 0, 1], [0, 1, 1, 0, 1, 0], [1, 1, 0, 0, 0, 1], [0, 0, 0, 1, 1, 1]], np.uint8)
    c, sc, wd = o.mixfp4_quantize(w, s2, tmap, 8, 64)
    assert np.array_equal(o.mixfp4_dequantize(c, sc, s2, tmap, 8, 64), wd)
    codes = np.zeros((1, 8), np.uint8)
    codes[0, 0] = 0xF7          # elements 0, 1: codes 0x7, 0xF
    codes[0, 1] = 0x08          # element 2: code 0x8
    scales = np.full((1, 1), 0x38, np.uint8)
    for e0, big in ((1, 7.0), (0, 6.0)):
        d = bf16_float(o.mixfp4_dequantize(codes, scales, S2_POW2, np.array([[e0]], np.uint8), 1, 16))
        assert d[0, 0] == big * 2.0 ** -10 and d[0, 1] == -big * 2.0 ** -10
        assert d[0, 2] == 0.0 and np.signbit(d[0, 2]) and not np.signbit(d[0, 3])


# ---------------------------------------------------------------------------
# the NVFP4 linear layer Y = X' W'^T
# ---------------------------------------------------------------------------

def check_linear_closed_forms(o):
    """Codes 1.0 (0x2) and -1.0 (0xA) with scale 1 (0x38): every output is
    +-K * s2x[t] * s2w; Yabs = K * s2x[t] * s2w."""
    K = 48
    xc = np.full((3, K // 2), 0x22, np.uint8)
    xs = np.full((3, K // 16), 0x38, np.uint8)
    wc = np.full((2, K // 2), 0x22, np.uint8)
    wc[1] = 0xAA
    ws = np.full((2, K // 16), 0x38, np.uint8)
    s2x = np.float32([1.0, 0.25, 3.0])
    y, ya = o.nvfp4_linear(xc, xs, s2x, wc, ws, np.float32(0.5))
    want = K * s2x.astype(np.float64)[:, None] * 0.5 * np.array([1.0, -1.0])
    assert np.array_equal(y, want) and np.array_equal(ya, np.abs(want))
    # one s2 for all rows
    y1, _ = o.nvfp4_linear(xc, xs, np.float32(2.0), wc, ws, np.float32(0.5))
    assert np.array_equal(y1, K * 2.0 * 0.5 * np.array([[1.0, -1.0]] * 3))


def check_linear_fixed_points(o):
    """Weights and activations built as NVFP4 fixed points (w = c*S*s2, every
    E4M3 scale): the pinned quantizer returns their codes and scales, and the
    layer on those equals numpy's float64 product X @ W.T of the original
    values exactly (K = 64 keeps every partial sum exact in binary64).  A
    transposed operand, a wrong scale or nibble index, or a dropped or
    misplaced s2 all change it."""
    rng = np.random.default_rng(120)
    _, _, _, wb = _fixed_point_case(rng, n_rows=119, nb=4)
    wc, wsc, _ = o.quantize(wb, None, None, S2_POW2, dequant=False)
    # activations: per-token s2 = 2^-10 * 2^(t mod 5), a random scale per
    # block, and one |c| = 6 per block so each block is a fixed point
    _, _, codes_x, _ = _fixed_point_case(rng, n_rows=119, nb=4)
    sb = rng.integers(0x08, 0x7F, (119, 4)).astype(np.uint8)
    S = np.repeat(torch_e4m3_value(sb).astype(np.float64), 16, axis=1)
    s2x = (float(S2_POW2) * np.exp2(np.arange(119) % 5)).astype(np.float32)
    x = code_value(codes_x) * S * s2x[:, None].astype(np.float64)
    xb = torch_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_float(xb).astype(np.float64), x)
    xc = np.empty((119, 32), np.uint8)
    xsc = np.empty((119, 4), np.uint8)
    for t in range(119):
        c, sc_, _ = o.quantize(xb[t:t + 1], None, None, s2x[t], dequant=False)
        xc[t], xsc[t] = c[0], sc_[0]
    assert np.array_equal(xsc, sb)
    y, ya = o.nvfp4_linear(xc, xsc, s2x, wc, wsc, S2_POW2)
    xf, wf = bf16_float(xb).astype(np.float64), bf16_float(wb).astype(np.float64)
    assert np.array_equal(y, xf @ wf.T)
    assert np.array_equal(ya, np.abs(xf) @ np.abs(wf).T)
    # rows and columns are independent: a slice gives the same entries
    y2, _ = o.nvfp4_linear(xc[5:9], xsc[5:9], s2x[5:9], wc[17:30], wsc[17:30], S2_POW2)
    assert np.array_equal(y2, y[5:9, 17:30])


ALL_CHECKS = [
    check_e2m1_table, check_e2m1_nearest_dense, check_e4m3_vs_torch, check_e4m3_decode_vs_torch,
    check_bf16_vs_torch, check_sigmoid, check_expf_correctly_rounded, check_tensor_scale,
    check_fixed_points, check_block_factor_m, check_subblock_logits, check_zero_blocks, check_clamps,
    check_s2_zero, check_amax_block_closed_form, check_error_bound, check_monotone,
    check_plain_rtn_reduction, check_dequantize_roundtrip, check_act_per_token,
    check_fo6_four_fixed_points, check_fo6_six_fixed_points, check_fo6_ties_keep_six,
    check_fo6_never_worse_than_rtn, check_mx_scale_closed_forms, check_mx_fixed_points,
    check_mx_factor_and_subblocks, check_mx_plain_reduction, check_e0m3_levels, check_mixfp4_maps,
    check_linear_closed_forms, check_linear_fixed_points, check_mixfp4_dequantize,
    check_fo6_zero_and_act,
]
