"""ctypes loader of libfocus_nvfp4.so (built in-tree by ``build.py``).

The C signatures mirror include/focus_nvfp4.h: device pointers and sizes as
integers, the stream as a ``hipStream_t`` handle (``void*``).  There is no
fallback: a missing library raises ``FocusLibraryMissing``.
"""
from __future__ import annotations

import ctypes as ct
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfocus_nvfp4.so")

_VP = ct.c_void_p
_I64 = ct.c_int64
_INT = ct.c_int

class ScaleDesc(ct.Structure):
    _fields_ = [("w_bf16", _VP), ("numel", _I64), ("s2_out", _VP), ("amax_out", _VP)]


class QuantDesc(ct.Structure):
    _fields_ = [("w_bf16", _VP), ("rows", _I64), ("cols", _I64), ("m", _VP), ("q", _VP),
                ("s2", _VP), ("codes", _VP), ("scales", _VP), ("w_deq", _VP)]


class DequantDesc(ct.Structure):
    _fields_ = [("codes", _VP), ("scales", _VP), ("s2", _VP), ("s2_per_row", _INT),
                ("rows", _I64), ("cols", _I64), ("out", _VP)]


class MixDesc(ct.Structure):
    _fields_ = [("w_bf16", _VP), ("rows", _I64), ("cols", _I64), ("s2", _VP), ("map", _VP),
                ("tile_rows", _I64), ("tile_cols", _I64), ("codes", _VP), ("scales", _VP),
                ("w_deq", _VP)]


class LinearWeight(ct.Structure):
    _fields_ = [("w_codes", _VP), ("w_scales", _VP), ("w_s2", _VP), ("N", _I64), ("y", _VP)]


_SIGNATURES = {
    "focus_abi_version": (_INT, []),
    "focus_status_string": (ct.c_char_p, [_INT]),
    "focus_tensor_scale": (_INT, [_VP, _I64, _VP, _VP, _VP]),
    "focus_quantize": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "focus_dequantize": (_INT, [_VP, _VP, _VP, _INT, _I64, _I64, _VP, _VP]),
    "focus_quantize_act_per_token": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "focus_quantize_fo6": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "focus_quantize_act_per_token_fo6": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "focus_tensor_scale_many": (_INT, [ct.POINTER(ScaleDesc), _INT, _VP]),
    "focus_quantize_many": (_INT, [ct.POINTER(QuantDesc), _INT, _VP]),
    "focus_dequantize_many": (_INT, [ct.POINTER(DequantDesc), _INT, _VP]),
    "focus_quantize_fo6_many": (_INT, [ct.POINTER(QuantDesc), _INT, _VP]),
    "focus_quantize_mx": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP]),
    "focus_quantize_mx_many": (_INT, [ct.POINTER(QuantDesc), _INT, _VP]),
    "focus_dequantize_mx": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP]),
    "focus_quantize_mixfp4": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _I64, _VP, _VP, _VP, _VP]),
    "focus_quantize_mixfp4_many": (_INT, [ct.POINTER(MixDesc), _INT, _VP]),
    "focus_dequantize_mixfp4": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _VP, _VP]),
    "focus_nvfp4_linear": (_INT, [_VP, _VP, _VP, _INT, _I64, _VP, _VP, _VP, _I64, _I64, _VP, _INT, _VP, _I64,
                                  _VP]),
    "focus_nvfp4_linear_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "focus_nvfp4_linear_grouped": (_INT, [_VP, _VP, _VP, _INT, _I64, _I64, ct.POINTER(LinearWeight), _INT, _INT,
                                          _VP, _I64, _VP]),
    "focus_nvfp4_linear_noalloc": (_INT, [_VP, _VP, _VP, _INT, _I64, _VP, _VP, _VP, _I64, _I64, _VP, _INT,
                                          _VP]),
    "focus_nvfp4_linear_scratch_bytes": (_I64, []),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class FocusLibraryMissing(RuntimeError):
    pass


class FocusError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfocus_nvfp4 status {status}: {message}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FocusLibraryMissing(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ct.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = lib().focus_status_string(status).decode()
        raise FocusError(status, msg)
