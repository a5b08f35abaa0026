"""Python access to the scalar CPU oracle of the FOCUS NVFP4 quantizer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product path never imports it.

Arrays are numpy: BF16 data travels as its uint16 bit patterns, FP32 as
float32, codes and scale bytes as uint8.  Every method is a thin ctypes call
into ``focus_oracle.c``; the arithmetic lives there.  ctypes releases the GIL
during a call, so callers may run row ranges on several threads.

``Oracle(path)`` wraps one build of the library; the module-level functions
use the default build ``oracle/liboracle.so`` (built on first use).
"""
import ctypes as _ct
import os as _os

import numpy as _np

_HERE = _os.path.dirname(_os.path.abspath(__file__))
LIB_PATH = _os.path.join(_HERE, "liboracle.so")

_u16p = _ct.POINTER(_ct.c_uint16)
_u8p = _ct.POINTER(_ct.c_uint8)
_f32p = _ct.POINTER(_ct.c_float)
_f64p = _ct.POINTER(_ct.c_double)
_i64 = _ct.c_int64
_f = _ct.c_float

_SIGNATURES = {
    "oracle_abi_version": (_ct.c_int, []),
    "oracle_bf16_value": (_f, [_ct.c_uint16]),
    "oracle_e2m1_value": (_f, [_ct.c_uint]),
    "oracle_e2m1_round": (_ct.c_uint, [_f]),
    "oracle_e4m3_value": (_f, [_ct.c_uint]),
    "oracle_e4m3_round": (_ct.c_uint, [_f]),
    "oracle_bf16_round": (_ct.c_uint16, [_f]),
    "oracle_expf": (_f, [_f]),
    "oracle_sigmoid": (_f, [_f]),
    "oracle_tensor_scale": (_f, [_u16p, _i64, _f32p]),
    "oracle_block_scale": (_ct.c_uint, [_f, _f, _f]),
    "oracle_element_code": (_ct.c_uint, [_ct.c_uint16, _f, _f, _f]),
    "oracle_dequant_value": (_ct.c_uint16, [_ct.c_uint, _f, _f]),
    "oracle_subblock_codes": (None, [_u16p, _ct.c_int, _f, _f, _f, _u8p]),
    "oracle_quantize": (None, [_u16p, _i64, _i64, _f32p, _f32p, _f, _u8p, _u8p, _u16p]),
    "oracle_dequantize": (None, [_u8p, _u8p, _f32p, _ct.c_int, _i64, _i64, _u16p]),
    "oracle_quantize_act_per_token": (None, [_u16p, _i64, _i64, _u8p, _u8p, _f32p, _u16p]),
    "oracle_e2m1_round_n": (None, [_f32p, _i64, _u8p]),
    "oracle_e4m3_round_n": (None, [_f32p, _i64, _u8p]),
    "oracle_bf16_round_n": (None, [_f32p, _i64, _u16p]),
    "oracle_sigmoid_n": (None, [_f32p, _i64, _f32p]),
    "oracle_expf_n": (None, [_f32p, _i64, _f32p]),
    "oracle_fo6_block": (_ct.c_uint, [_u16p, _f, _u8p]),
    "oracle_e8m0_value": (_f, [_ct.c_uint]),
    "oracle_e0m3_round": (_ct.c_uint, [_f]),
    "oracle_e0m3_value": (_f, [_ct.c_uint]),
    "oracle_mixfp4_quantize": (None, [_u16p, _i64, _i64, _f, _u8p, _i64, _i64, _u8p, _u8p, _u16p]),
    "oracle_mx_block_scale": (_ct.c_uint, [_f, _f]),
    "oracle_mx_quantize": (None, [_u16p, _i64, _i64, _f32p, _f32p, _u8p, _u8p, _u16p]),
    "oracle_mx_dequantize": (None, [_u8p, _u8p, _i64, _i64, _u16p]),
    "oracle_fo6_quantize": (None, [_u16p, _i64, _i64, _f32p, _ct.c_int, _u8p, _u8p, _u16p]),
    "oracle_fo6_quantize_act_per_token": (None, [_u16p, _i64, _i64, _u8p, _u8p, _f32p, _u16p]),
    "oracle_mixfp4_dequantize": (None, [_u8p, _u8p, _f, _u8p, _i64, _i64, _i64, _i64, _u16p]),
    "oracle_nvfp4_linear": (None, [_u8p, _u8p, _f32p, _ct.c_int, _i64, _u8p, _u8p, _f32p, _i64, _i64,
                                   _f64p, _f64p]),
}


def _ptr(a, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctype)


def _as(a, dtype):
    a = _np.ascontiguousarray(a)
    assert a.dtype == dtype, f"expected {dtype}, got {a.dtype}"
    return a


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str = LIB_PATH):
        lib = _ct.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        self.lib = lib
        self.path = path

    # ---- scalar helpers ----------------------------------------------------
    def bf16_value(self, h):
        return self.lib.oracle_bf16_value(int(h))

    def e2m1_value(self, code):
        return self.lib.oracle_e2m1_value(int(code))

    def e2m1_round(self, x):
        return self.lib.oracle_e2m1_round(float(x))

    def e4m3_value(self, b):
        return self.lib.oracle_e4m3_value(int(b))

    def e4m3_round(self, t):
        return self.lib.oracle_e4m3_round(float(t))

    def bf16_round(self, x):
        return self.lib.oracle_bf16_round(float(x))

    def expf(self, x):
        return self.lib.oracle_expf(float(x))

    def sigmoid(self, q):
        return self.lib.oracle_sigmoid(float(q))

    def block_scale(self, a, mb, s2):
        return self.lib.oracle_block_scale(float(a), float(mb), float(s2))

    def element_code(self, w_bits, S, sig, s2):
        return self.lib.oracle_element_code(int(w_bits), float(S), float(sig), float(s2))

    def dequant_value(self, code, S, s2):
        return self.lib.oracle_dequant_value(int(code), float(S), float(s2))

    # ---- array forms (loops run in C) ---------------------------------------
    def e2m1_round_array(self, x):
        x = _as(x, _np.float32).ravel()
        out = _np.empty(x.size, _np.uint8)
        self.lib.oracle_e2m1_round_n(_ptr(x, _f32p), x.size, _ptr(out, _u8p))
        return out

    def e4m3_round_array(self, t):
        t = _as(t, _np.float32).ravel()
        out = _np.empty(t.size, _np.uint8)
        self.lib.oracle_e4m3_round_n(_ptr(t, _f32p), t.size, _ptr(out, _u8p))
        return out

    def bf16_round_array(self, x):
        x = _as(x, _np.float32).ravel()
        out = _np.empty(x.size, _np.uint16)
        self.lib.oracle_bf16_round_n(_ptr(x, _f32p), x.size, _ptr(out, _u16p))
        return out

    def sigmoid_array(self, q):
        q = _as(q, _np.float32).ravel()
        out = _np.empty(q.size, _np.float32)
        self.lib.oracle_sigmoid_n(_ptr(q, _f32p), q.size, _ptr(out, _f32p))
        return out

    def expf_array(self, x):
        x = _as(x, _np.float32).ravel()
        out = _np.empty(x.size, _np.float32)
        self.lib.oracle_expf_n(_ptr(x, _f32p), x.size, _ptr(out, _f32p))
        return out

    def subblock_codes(self, w_bits, S, sig, s2):
        w_bits = _as(w_bits, _np.uint16).ravel()
        out = _np.empty(w_bits.size, _np.uint8)
        self.lib.oracle_subblock_codes(_ptr(w_bits, _u16p), int(w_bits.size), float(S),
                                       float(sig), float(s2), _ptr(out, _u8p))
        return out

    # ---- the method -----------------------------------------------------------
    def tensor_scale(self, w_bits):
        """(s2, amax) of the BF16 bit patterns ``w_bits`` (any shape)."""
        w_bits = _as(w_bits, _np.uint16)
        amax = _ct.c_float(0.0)
        s2 = self.lib.oracle_tensor_scale(_ptr(w_bits, _u16p), int(w_bits.size),
                                          _ct.byref(amax))
        return _np.float32(s2), _np.float32(amax.value)

    def quantize(self, w_bits, m, q, s2, dequant=True):
        """W [rows, cols] (uint16 BF16 bits), m [rows, cols/16] or None,
        q [rows, cols/8] or None, scalar s2 -> (codes, scales, wdeq or None)."""
        w_bits = _as(w_bits, _np.uint16)
        rows, cols = w_bits.shape
        assert cols % 16 == 0
        if m is not None:
            m = _as(m, _np.float32)
            assert m.shape == (rows, cols // 16)
        if q is not None:
            q = _as(q, _np.float32)
            assert q.shape == (rows, cols // 8)
        codes = _np.empty((rows, cols // 2), _np.uint8)
        scales = _np.empty((rows, cols // 16), _np.uint8)
        wdeq = _np.empty((rows, cols), _np.uint16) if dequant else None
        self.lib.oracle_quantize(_ptr(w_bits, _u16p), rows, cols, _ptr(m, _f32p),
                                 _ptr(q, _f32p), float(s2), _ptr(codes, _u8p),
                                 _ptr(scales, _u8p), _ptr(wdeq, _u16p))
        return codes, scales, wdeq

    def dequantize(self, codes, scales, s2, s2_per_row=False):
        codes = _as(codes, _np.uint8)
        scales = _as(scales, _np.uint8)
        rows, half = codes.shape
        cols = 2 * half
        assert scales.shape == (rows, cols // 16)
        s2 = _np.ascontiguousarray(_np.atleast_1d(_np.asarray(s2, _np.float32)))
        assert s2.size >= (rows if s2_per_row else 1)
        out = _np.empty((rows, cols), _np.uint16)
        self.lib.oracle_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), _ptr(s2, _f32p),
                                   1 if s2_per_row else 0, rows, cols, _ptr(out, _u16p))
        return out

    def quantize_act_per_token(self, x_bits, dequant=False):
        """X [tokens, hidden] BF16 bits -> (codes, scales, s2 [tokens], xdeq or None)."""
        x_bits = _as(x_bits, _np.uint16)
        t, h = x_bits.shape
        assert h % 16 == 0
        codes = _np.empty((t, h // 2), _np.uint8)
        scales = _np.empty((t, h // 16), _np.uint8)
        s2 = _np.empty(t, _np.float32)
        xdeq = _np.empty((t, h), _np.uint16) if dequant else None
        self.lib.oracle_quantize_act_per_token(_ptr(x_bits, _u16p), t, h, _ptr(codes, _u8p),
                                               _ptr(scales, _u8p), _ptr(s2, _f32p),
                                               _ptr(xdeq, _u16p))
        return codes, scales, s2, xdeq


    # ---- FourOverSix -------------------------------------------------------------
    def fo6_quantize(self, w_bits, s2, s2_per_row=False, dequant=True):
        """FourOverSix RTN of [rows, cols]: one s2 (weights) or s2 per row."""
        w_bits = _as(w_bits, _np.uint16)
        rows, cols = w_bits.shape
        assert cols % 16 == 0
        s2 = _np.ascontiguousarray(_np.atleast_1d(_np.asarray(s2, _np.float32)))
        assert s2.size >= (rows if s2_per_row else 1)
        codes = _np.empty((rows, cols // 2), _np.uint8)
        scales = _np.empty((rows, cols // 16), _np.uint8)
        wdeq = _np.empty((rows, cols), _np.uint16) if dequant else None
        self.lib.oracle_fo6_quantize(_ptr(w_bits, _u16p), rows, cols, _ptr(s2, _f32p),
                                     1 if s2_per_row else 0, _ptr(codes, _u8p),
                                     _ptr(scales, _u8p), _ptr(wdeq, _u16p))
        return codes, scales, wdeq

    def fo6_quantize_act_per_token(self, x_bits, dequant=False):
        x_bits = _as(x_bits, _np.uint16)
        t, h = x_bits.shape
        assert h % 16 == 0
        codes = _np.empty((t, h // 2), _np.uint8)
        scales = _np.empty((t, h // 16), _np.uint8)
        s2 = _np.empty(t, _np.float32)
        xdeq = _np.empty((t, h), _np.uint16) if dequant else None
        self.lib.oracle_fo6_quantize_act_per_token(_ptr(x_bits, _u16p), t, h, _ptr(codes, _u8p),
                                                   _ptr(scales, _u8p), _ptr(s2, _f32p),
                                                   _ptr(xdeq, _u16p))
        return codes, scales, s2, xdeq

    # ---- FOCUS on MXFP4 ---------------------------------------------------------
    def e8m0_value(self, b):
        return self.lib.oracle_e8m0_value(int(b))

    def mx_block_scale(self, a, mb=1.0):
        return self.lib.oracle_mx_block_scale(float(a), float(mb))

    def mx_quantize(self, w_bits, m, q, dequant=True):
        """FOCUS on MXFP4: W [rows, cols] (cols % 32 == 0), m [rows, cols/32] or
        None, q [rows, cols/8] or None -> (codes, E8M0 scales [rows, cols/32],
        wdeq or None)."""
        w_bits = _as(w_bits, _np.uint16)
        rows, cols = w_bits.shape
        assert cols % 32 == 0
        if m is not None:
            m = _as(m, _np.float32)
            assert m.shape == (rows, cols // 32)
        if q is not None:
            q = _as(q, _np.float32)
            assert q.shape == (rows, cols // 8)
        codes = _np.empty((rows, cols // 2), _np.uint8)
        scales = _np.empty((rows, cols // 32), _np.uint8)
        wdeq = _np.empty((rows, cols), _np.uint16) if dequant else None
        self.lib.oracle_mx_quantize(_ptr(w_bits, _u16p), rows, cols, _ptr(m, _f32p), _ptr(q, _f32p),
                                    _ptr(codes, _u8p), _ptr(scales, _u8p), _ptr(wdeq, _u16p))
        return codes, scales, wdeq

    def mx_dequantize(self, codes, scales):
        codes = _as(codes, _np.uint8)
        scales = _as(scales, _np.uint8)
        rows, half = codes.shape
        cols = 2 * half
        assert scales.shape == (rows, cols // 32)
        out = _np.empty((rows, cols), _np.uint16)
        self.lib.oracle_mx_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), rows, cols, _ptr(out, _u16p))
        return out

    # ---- FlipQuant MixFP4 --------------------------------------------------------
    def e0m3_round(self, x):
        return self.lib.oracle_e0m3_round(float(x))

    def e0m3_value(self, code):
        return self.lib.oracle_e0m3_value(int(code))

    def mixfp4_quantize(self, w_bits, s2, tile_map, tile_rows, tile_cols=64, dequant=True):
        """MixFP4: W [rows, cols], per-tensor s2, tile_map [rows/tile_rows,
        cols/tile_cols] (nonzero = E0M3 tile, else E2M1 with FourOverSix)."""
        w_bits = _as(w_bits, _np.uint16)
        rows, cols = w_bits.shape
        assert cols % 16 == 0 and rows % tile_rows == 0 and cols % tile_cols == 0
        tile_map = _as(_np.asarray(tile_map).astype(_np.uint8), _np.uint8)
        assert tile_map.shape == (rows // tile_rows, cols // tile_cols)
        codes = _np.empty((rows, cols // 2), _np.uint8)
        scales = _np.empty((rows, cols // 16), _np.uint8)
        wdeq = _np.empty((rows, cols), _np.uint16) if dequant else None
        self.lib.oracle_mixfp4_quantize(_ptr(w_bits, _u16p), rows, cols, float(s2), _ptr(tile_map, _u8p),
                                        tile_rows, tile_cols, _ptr(codes, _u8p), _ptr(scales, _u8p),
                                        _ptr(wdeq, _u16p))
        return codes, scales, wdeq

    def mixfp4_dequantize(self, codes, scales, s2, tile_map, tile_rows, tile_cols=64):
        """Stored MixFP4 [rows, cols] -> BF16 bits (E0M3 or E2M1 per tile)."""
        codes, scales = _as(codes, _np.uint8), _as(scales, _np.uint8)
        rows, cols = codes.shape[0], 2 * codes.shape[1]
        assert scales.shape == (rows, cols // 16) and rows % tile_rows == 0 and cols % tile_cols == 0
        tile_map = _as(_np.asarray(tile_map).astype(_np.uint8), _np.uint8)
        assert tile_map.shape == (rows // tile_rows, cols // tile_cols)
        out = _np.empty((rows, cols), _np.uint16)
        self.lib.oracle_mixfp4_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), float(s2), _ptr(tile_map, _u8p),
                                          rows, cols, tile_rows, tile_cols, _ptr(out, _u16p))
        return out

    def nvfp4_linear(self, x_codes, x_scales, x_s2, w_codes, w_scales, w_s2):
        """Y = X' W'^T of NVFP4 activations X [M, K] (s2 per token, or one
        value) and NVFP4 weights W [N, K] (one s2): returns (Y, Yabs) in
        float64, Yabs the matching sum of |products| (error-bound scale)."""
        x_codes, x_scales = _as(x_codes, _np.uint8), _as(x_scales, _np.uint8)
        w_codes, w_scales = _as(w_codes, _np.uint8), _as(w_scales, _np.uint8)
        M, K = x_codes.shape[0], 2 * x_codes.shape[1]
        N = w_codes.shape[0]
        assert K % 16 == 0 and w_codes.shape[1] * 2 == K
        assert x_scales.shape == (M, K // 16) and w_scales.shape == (N, K // 16)
        xs2 = _np.ascontiguousarray(_np.atleast_1d(_np.asarray(x_s2, _np.float32)))
        ws2 = _np.ascontiguousarray(_np.atleast_1d(_np.asarray(w_s2, _np.float32)))
        assert xs2.size in (1, M) and ws2.size == 1
        y = _np.empty((M, N), _np.float64)
        yabs = _np.empty((M, N), _np.float64)
        self.lib.oracle_nvfp4_linear(_ptr(x_codes, _u8p), _ptr(x_scales, _u8p), _ptr(xs2, _f32p),
                                     1 if xs2.size == M else 0, M, _ptr(w_codes, _u8p),
                                     _ptr(w_scales, _u8p), _ptr(ws2, _f32p), N, K, _ptr(y, _f64p),
                                     _ptr(yabs, _f64p))
        return y, yabs


_default = None


def default() -> Oracle:
    """The default build, compiled with gcc on first use if missing."""
    global _default
    if _default is None:
        if not _os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        _default = Oracle(LIB_PATH)
    return _default


def __getattr__(name):
    # module-level access to the default build: oracle.quantize(...), ...
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
