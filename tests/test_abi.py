"""The C ABI: the library loads, exports every symbol include/*.h declares,
and rejects bad arguments on the host before any HIP call (CPU only: no
call here reaches a kernel launch)."""
import ctypes as ct
import glob
import os
import re

import pytest

from fp4_post_weight_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# status codes of include/focus_nvfp4.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_HIP, ERR_RANGE = 0, 1, 2, 3, 4, 5

FAKE = 0x10000  # a 64 KiB-aligned address that is never dereferenced


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(focus_[a-z0-9_]+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfocus_nvfp4.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"focus_tensor_scale", "focus_quantize", "focus_dequantize",
            "focus_quantize_act_per_token"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert names <= set(_lib.EXPORTED), "binding does not wrap every declared call"


def test_version_and_status_strings(lib):
    assert lib.focus_abi_version() == 1
    for s in range(6):
        assert lib.focus_status_string(s)
    assert lib.focus_status_string(99) == b"unknown status"


def test_quantize_validation(lib):
    q = lib.focus_quantize
    # null required pointers
    assert q(None, 4, 32, None, None, FAKE, FAKE, FAKE, None, None) == ERR_NULL
    assert q(FAKE, 4, 32, None, None, None, FAKE, FAKE, None, None) == ERR_NULL
    assert q(FAKE, 4, 32, None, None, FAKE, None, FAKE, None, None) == ERR_NULL
    assert q(FAKE, 4, 32, None, None, FAKE, FAKE, None, None, None) == ERR_NULL
    # shapes
    assert q(FAKE, 4, 24, None, None, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert q(FAKE, -1, 32, None, None, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert q(FAKE, 4, -16, None, None, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert q(FAKE, 1 << 40, 1 << 40, None, None, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    # alignment
    assert q(FAKE + 2, 4, 32, None, None, FAKE, FAKE, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 4, 32, FAKE + 2, None, FAKE, FAKE, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 4, 32, None, FAKE + 4, FAKE, FAKE, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 4, 32, None, None, FAKE + 1, FAKE, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 4, 32, None, None, FAKE, FAKE + 4, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 4, 32, None, None, FAKE, FAKE, FAKE, FAKE + 8, None) == ERR_ALIGN
    # empty tensors are a no-op, even with null pointers
    assert q(None, 0, 32, None, None, None, None, None, None, None) == OK
    assert q(None, 5, 0, None, None, None, None, None, None, None) == OK


def test_dequantize_validation(lib):
    d = lib.focus_dequantize
    assert d(None, FAKE, FAKE, 0, 2, 32, FAKE, None) == ERR_NULL
    assert d(FAKE, None, FAKE, 0, 2, 32, FAKE, None) == ERR_NULL
    assert d(FAKE, FAKE, None, 0, 2, 32, FAKE, None) == ERR_NULL
    assert d(FAKE, FAKE, FAKE, 0, 2, 32, None, None) == ERR_NULL
    assert d(FAKE, FAKE, FAKE, 0, 2, 40, FAKE, None) == ERR_SHAPE
    assert d(FAKE, FAKE, FAKE, 2, 2, 32, FAKE, None) == ERR_RANGE
    assert d(FAKE + 4, FAKE, FAKE, 0, 2, 32, FAKE, None) == ERR_ALIGN
    assert d(FAKE, FAKE, FAKE, 0, 2, 32, FAKE + 8, None) == ERR_ALIGN
    assert d(None, None, None, 0, 0, 32, None, None) == OK


def test_tensor_scale_validation(lib):
    t = lib.focus_tensor_scale
    assert t(FAKE, 10, None, None, None) == ERR_NULL
    assert t(None, 10, FAKE, None, None) == ERR_NULL
    assert t(FAKE, -1, FAKE, None, None) == ERR_SHAPE
    assert t(FAKE + 8, 10, FAKE, None, None) == ERR_ALIGN
    assert t(FAKE, 10, FAKE + 2, None, None) == ERR_ALIGN
    assert t(FAKE, 10, FAKE, FAKE + 1, None) == ERR_ALIGN


def test_act_validation(lib):
    a = lib.focus_quantize_act_per_token
    assert a(None, 4, 64, FAKE, FAKE, FAKE, None, None) == ERR_NULL
    assert a(FAKE, 4, 64, None, FAKE, FAKE, None, None) == ERR_NULL
    assert a(FAKE, 4, 64, FAKE, None, FAKE, None, None) == ERR_NULL
    assert a(FAKE, 4, 64, FAKE, FAKE, None, None, None) == ERR_NULL
    assert a(FAKE, 4, 60, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert a(FAKE, 1 << 32, 16, FAKE, FAKE, FAKE, None, None) == ERR_RANGE
    assert a(FAKE, 4, 64, FAKE + 4, FAKE, FAKE, None, None) == ERR_ALIGN
    assert a(FAKE, 4, 64, FAKE, FAKE, FAKE, FAKE + 8, None) == ERR_ALIGN
    assert a(None, 0, 64, None, None, None, None, None) == OK


def test_binding_refuses_cpu_tensors():
    import torch

    import fp4_post_weight_amd as focus
    w = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        focus.quantize(w)
    with pytest.raises(TypeError):
        focus.tensor_scale(torch.zeros(4, dtype=torch.float32))


def test_product_path_does_not_reach_the_oracle():
    """The package and its sources never import or load the oracle."""
    pkg = os.path.join(ROOT, "fp4_post_weight_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if path.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(path).read()
            assert "oracle" not in text.replace("Oracle", "").lower().replace("no oracle", ""), path


def test_batched_validation(lib):
    QD, SD, DD = _lib.QuantDesc, _lib.ScaleDesc, _lib.DequantDesc
    assert lib.focus_quantize_many(None, 0, None) == OK
    assert lib.focus_quantize_many(None, 2, None) == ERR_NULL
    assert lib.focus_quantize_many((QD * 1)(), -1, None) == ERR_RANGE
    good = QD(FAKE, 4, 32, None, None, FAKE, FAKE, FAKE, None)
    bad_shape = QD(FAKE, 4, 24, None, None, FAKE, FAKE, FAKE, None)
    bad_align = QD(FAKE, 4, 32, None, None, FAKE, FAKE + 4, FAKE, None)
    empty = QD(None, 0, 32, None, None, None, None, None, None)
    # every descriptor is checked before anything is launched
    assert lib.focus_quantize_many((QD * 3)(good, empty, bad_shape), 3, None) == ERR_SHAPE
    assert lib.focus_quantize_many((QD * 2)(bad_align, good), 2, None) == ERR_ALIGN
    assert lib.focus_quantize_many((QD * 2)(empty, empty), 2, None) == OK
    assert lib.focus_tensor_scale_many(None, 1, None) == ERR_NULL
    assert lib.focus_tensor_scale_many((SD * 2)(SD(FAKE, 8, FAKE, None), SD(FAKE, 8, None, None)), 2,
                                       None) == ERR_NULL
    assert lib.focus_tensor_scale_many((SD * 1)(SD(FAKE, -3, FAKE, None)), 1, None) == ERR_SHAPE
    assert lib.focus_dequantize_many((DD * 1)(DD(FAKE, FAKE, FAKE, 3, 2, 32, FAKE)), 1, None) == ERR_RANGE
    assert lib.focus_dequantize_many((DD * 1)(DD(FAKE, FAKE, FAKE, 0, 2, 32, FAKE + 2)), 1, None) == ERR_ALIGN
    assert lib.focus_dequantize_many(None, 0, None) == OK


def test_descriptor_layout():
    """ctypes mirrors of the C descriptor structs (LP64 layout)."""
    assert ct.sizeof(_lib.QuantDesc) == 9 * 8
    assert ct.sizeof(_lib.ScaleDesc) == 4 * 8
    assert ct.sizeof(_lib.DequantDesc) == 7 * 8
    assert _lib.DequantDesc.rows.offset == 32


def test_fo6_validation(lib):
    QD = _lib.QuantDesc
    assert lib.focus_quantize_fo6(None, 4, 32, FAKE, FAKE, FAKE, None, None) == ERR_NULL
    assert lib.focus_quantize_fo6(FAKE, 4, 30, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert lib.focus_quantize_fo6(FAKE, 0, 32, None, None, None, None, None) == OK
    with_m = QD(FAKE, 4, 32, FAKE, None, FAKE, FAKE, FAKE, None)
    assert lib.focus_quantize_fo6_many((QD * 1)(with_m), 1, None) == ERR_RANGE
    assert lib.focus_quantize_act_per_token_fo6(FAKE, 4, 64, None, FAKE, FAKE, None, None) == ERR_NULL
    assert lib.focus_quantize_act_per_token_fo6(FAKE + 2, 4, 64, FAKE, FAKE, FAKE, None, None) == ERR_ALIGN


def test_mx_validation(lib):
    QD = _lib.QuantDesc
    q = lib.focus_quantize_mx
    assert q(FAKE, 4, 48, None, None, FAKE, FAKE, None, None) == ERR_SHAPE  # cols % 32
    assert q(None, 4, 64, None, None, FAKE, FAKE, None, None) == ERR_NULL
    assert q(FAKE, 4, 64, None, None, FAKE + 4, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 0, 64, None, None, None, None, None, None) == OK
    assert lib.focus_quantize_mx_many((QD * 1)(QD(FAKE, 4, 48, None, None, None, FAKE, FAKE, None)), 1,
                                      None) == ERR_SHAPE
    assert lib.focus_dequantize_mx(FAKE, FAKE, 2, 48, FAKE, None) == ERR_SHAPE
    assert lib.focus_dequantize_mx(FAKE, None, 2, 64, FAKE, None) == ERR_NULL


def test_mixfp4_validation(lib):
    MD = _lib.MixDesc
    q = lib.focus_quantize_mixfp4
    #        w     rows cols s2    map   th  tw  codes scales deq
    assert q(FAKE, 16, 128, FAKE, FAKE, 0, 64, FAKE, FAKE, None, None) == ERR_SHAPE   # tile_rows < 1
    assert q(FAKE, 16, 128, FAKE, FAKE, 8, 8, FAKE, FAKE, None, None) == ERR_SHAPE    # tile_cols < 16
    assert q(FAKE, 16, 128, FAKE, FAKE, 8, 40, FAKE, FAKE, None, None) == ERR_SHAPE   # not a multiple of 16
    assert q(FAKE, 12, 128, FAKE, FAKE, 8, 64, FAKE, FAKE, None, None) == ERR_SHAPE   # rows % tile_rows
    assert q(FAKE, 16, 160, FAKE, FAKE, 8, 64, FAKE, FAKE, None, None) == ERR_SHAPE   # cols % tile_cols
    assert q(FAKE, 1 << 24, 2048, FAKE, FAKE, 8, 64, FAKE, FAKE, None, None) == ERR_RANGE  # 2^31 blocks
    assert q(FAKE, 16, 128, FAKE, None, 8, 64, FAKE, FAKE, None, None) == ERR_NULL
    assert q(FAKE, 16, 128, None, FAKE, 8, 64, FAKE, FAKE, None, None) == ERR_NULL
    assert q(FAKE + 2, 16, 128, FAKE, FAKE, 8, 64, FAKE, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 16, 128, FAKE, FAKE, 8, 64, FAKE + 4, FAKE, None, None) == ERR_ALIGN
    assert q(FAKE, 16, 128, FAKE, FAKE, 8, 64, FAKE, FAKE, FAKE + 8, None) == ERR_ALIGN
    assert q(None, 0, 128, None, None, 8, 64, None, None, None, None) == OK
    many = lib.focus_quantize_mixfp4_many
    good = MD(FAKE, 16, 128, FAKE, FAKE, 8, 64, FAKE, FAKE, None)
    bad = MD(FAKE, 16, 128, FAKE, FAKE, 16, 48, FAKE, FAKE, None)
    assert many((MD * 2)(good, bad), 2, None) == ERR_SHAPE
    assert many(None, 0, None) == OK
    assert many(None, 1, None) == ERR_NULL
    assert ct.sizeof(MD) == 10 * 8


def test_linear_validation(lib):
    g = lib.focus_nvfp4_linear

    def f(*args):  # the calls below: no workspace
        return g(*args[:-1], None, 0, args[-1])
    #        xc    xs    xs2 per  M   wc    ws    ws2   N   K   y    dt  stream
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 40, FAKE, 0, None) == ERR_SHAPE   # K % 16
    assert f(FAKE, FAKE, FAKE, 1, -1, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, (1 << 31) + 1, 64, FAKE, 0, None) == ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 2, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == ERR_RANGE
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 2, None) == ERR_RANGE
    assert f(FAKE, FAKE, FAKE, 1, 1 << 21, FAKE, FAKE, FAKE, 1 << 21, 16, FAKE, 0, None) == ERR_RANGE  # grid
    assert f(None, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == ERR_NULL
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, None, FAKE, 8, 64, FAKE, 0, None) == ERR_NULL
    assert f(FAKE, FAKE, None, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == ERR_NULL
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, None, 0, None) == ERR_NULL
    assert f(FAKE + 4, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, None) == ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE + 2, 0, None) == ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE + 1, 8, 64, FAKE, 0, None) == ERR_ALIGN
    assert f(None, None, None, 1, 0, None, None, None, 8, 64, None, 0, None) == OK    # empty
    assert f(None, None, None, 1, 4, None, None, None, 0, 64, None, 1, None) == OK


def test_mixfp4_dequantize_validation(lib):
    d = lib.focus_dequantize_mixfp4
    #        codes scales s2  map   rows cols th  tw  out   stream
    assert d(FAKE, FAKE, FAKE, FAKE, 16, 128, 8, 48, FAKE, None) == ERR_SHAPE
    assert d(FAKE, FAKE, FAKE, FAKE, 12, 128, 8, 64, FAKE, None) == ERR_SHAPE
    assert d(FAKE, FAKE, FAKE, None, 16, 128, 8, 64, FAKE, None) == ERR_NULL
    assert d(FAKE, FAKE, FAKE, FAKE, 16, 128, 8, 64, FAKE + 8, None) == ERR_ALIGN
    assert d(FAKE, FAKE, FAKE, FAKE, 1 << 24, 2048, 8, 64, FAKE, None) == ERR_RANGE
    assert d(None, None, None, None, 0, 128, 8, 64, None, None) == OK


def test_binding_has_every_call():
    """The Python binding exposes every C call under the same name without
    the focus_ prefix."""
    import fp4_post_weight_amd as focus
    for name in _lib.EXPORTED:
        assert hasattr(focus, name[len("focus_"):]), name
    assert focus.status_string(0) == "ok"


def test_linear_workspace(lib):
    g = lib.focus_nvfp4_linear
    # a negative size and a misaligned workspace are rejected before any launch
    assert g(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, FAKE, -4, None) == ERR_RANGE
    assert g(FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, 64, FAKE, 0, FAKE + 2, 64, None) == ERR_ALIGN
    ws = lib.focus_nvfp4_linear_workspace_bytes
    assert ws(0, 16, 16) == 0 and ws(16, 16, 0) == 0  # empty: no query needed
    # the split depends on the device's compute units; with no device the
    # query fails and is reported (-1), never replaced by a guess (the split
    # model itself is checked on the GPU, tests/test_gpu_linear.py)
    import torch
    if not torch.cuda.is_available():
        assert ws(8192, 14336, 4096) == -1
