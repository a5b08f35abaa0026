"""fp4_post_weight_amd -- the FOCUS NVFP4 quantizer on AMD MI355X (gfx950).

A thin binding over the C ABI of ``libfocus_nvfp4.so`` (declared in
``include/focus_nvfp4.h``): argument marshalling only.  Every step of the
quantizer runs in the library's HIP kernels; torch supplies device memory
(``torch.empty`` on the input's device) and the current HIP stream.  If the
library has not been built, every call raises ``FocusLibraryMissing``; there
is no fallback.

Calls (same names as the C ABI, without the ``focus_`` prefix):

* ``tensor_scale(w)`` -> (s2, amax), FP32 tensors of one element
* ``quantize(w, m=None, q=None, s2=None, dequant=True)``
  -> ``Quantized(codes, scales, w_deq, s2)``
* ``dequantize(codes, scales, s2)`` -> BF16 tensor
* ``quantize_act_per_token(x, dequant=False)``
  -> ``Quantized(codes, scales, x_deq, s2 [tokens])``
* ``tensor_scale_many``, ``quantize_many``, ``dequantize_many``: the batched
  calls (one launch per run of up to 32 tensors).  Each returns a ``Batch``
  whose descriptor array is built once; calling it again re-launches the same
  work on the current stream without rebuilding anything.
* FourOverSix: ``quantize_fo6``, ``quantize_fo6_many``,
  ``quantize_act_per_token_fo6``; FOCUS on MXFP4: ``quantize_mx``,
  ``quantize_mx_many``, ``dequantize_mx``; FlipQuant MixFP4:
  ``quantize_mixfp4``, ``quantize_mixfp4_many``, ``dequantize_mixfp4``; the
  NVFP4 linear layer: ``nvfp4_linear``, ``nvfp4_linear_grouped`` (several
  weights sharing one X); ``abi_version``, ``status_string``.

BF16 inputs are ``torch.bfloat16`` tensors; codes and scales are ``uint8``
([rows, cols/2] with element 2j in the low nibble, and [rows, cols/16] E4M3
bytes).
"""
from __future__ import annotations

from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import FocusError, FocusLibraryMissing, library_path  # noqa: F401

__all__ = ["tensor_scale", "quantize", "dequantize", "quantize_act_per_token", "Quantized",
           "quantize_fo6", "quantize_act_per_token_fo6", "quantize_fo6_many",
           "quantize_mixfp4", "quantize_mixfp4_many", "dequantize_mixfp4", "nvfp4_linear",
           "nvfp4_linear_workspace_bytes", "nvfp4_linear_grouped", "nvfp4_linear_noalloc", "nvfp4_linear_scratch_bytes",
           "quantize_mx", "quantize_mx_many", "dequantize_mx",
           "tensor_scale_many", "quantize_many", "dequantize_many", "Batch",
           "FocusError", "FocusLibraryMissing", "abi_version", "status_string", "library_path"]


class Quantized(NamedTuple):
    codes: torch.Tensor
    scales: torch.Tensor
    deq: Optional[torch.Tensor]
    s2: torch.Tensor


def status_string(status: int) -> str:
    """The library's description of a status code."""
    return _lib.lib().focus_status_string(int(status)).decode()


def abi_version() -> int:
    return _lib.lib().focus_abi_version()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_dev(name, t, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _p(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _check_buf(name, t, dtype, device, numel):
    """A caller-supplied buffer: a contiguous tensor of `dtype` on `device`
    holding exactly `numel` elements.  Raises before anything is launched."""
    _check_dev(name, t, dtype, device)
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} elements, expected {numel}")


def _quant_outs(out, rows, cols, dev, dequant, s2=None, s2_rows=0, scale_block=16, label="out",
                deq_optional=False):
    """Output buffers of a quantizer call: allocated when `out` is None,
    otherwise checked (codes [rows, cols/2], scales [rows, cols/scale_block],
    deq [rows, cols] when dequant, and s2 [s2_rows] FP32 when s2_rows > 0).
    With deq_optional (the batched calls), an entry without a deq buffer
    gets no w' even when dequant is set.  Returns (codes, scales, deq or
    None, s2)."""
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // scale_block), dtype=torch.uint8, device=dev)
        deq = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) if dequant else None
        if s2_rows:
            s2 = torch.empty((s2_rows,), dtype=torch.float32, device=dev)
        return codes, scales, deq, s2
    if not isinstance(out, Quantized):
        raise TypeError(f"{label} must be a Quantized tuple of buffers")
    _check_buf(f"{label}.codes", out.codes, torch.uint8, dev, rows * cols // 2)
    _check_buf(f"{label}.scales", out.scales, torch.uint8, dev, rows * cols // scale_block)
    deq = None
    if dequant and not (deq_optional and out.deq is None):
        if out.deq is None:
            raise ValueError(f"dequant=True needs {label}.deq")
        _check_buf(f"{label}.deq", out.deq, torch.bfloat16, dev, rows * cols)
        deq = out.deq
    if s2_rows:
        if out.s2 is None:
            raise ValueError(f"{label}.s2 is required")
        _check_buf(f"{label}.s2", out.s2, torch.float32, dev, s2_rows)
        s2 = out.s2
    return out.codes, out.scales, deq, s2


def tensor_scale(w: torch.Tensor, s2_out: Optional[torch.Tensor] = None,
                 amax_out: Optional[torch.Tensor] = None):
    """s2 = amax|W| / (6*448) (and amax) as one-element FP32 device tensors."""
    _check_dev("w", w, torch.bfloat16)
    dev = w.device
    if s2_out is None:
        s2_out = torch.empty(1, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    _check_dev("s2_out", s2_out, torch.float32, dev)
    _check_dev("amax_out", amax_out, torch.float32, dev)
    if s2_out.numel() < 1 or amax_out.numel() < 1:
        raise ValueError("s2_out and amax_out must hold one float each")
    _lib.check(_lib.lib().focus_tensor_scale(_p(w), w.numel(), _p(s2_out), _p(amax_out),
                                             _stream(w)))
    return s2_out, amax_out


def quantize(w: torch.Tensor, m: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
             s2: Optional[torch.Tensor] = None, dequant: bool = True,
             out: Optional[Quantized] = None) -> Quantized:
    """FOCUS quantizer of W [rows, cols] (BF16); m [rows, cols/16] FP32 or None
    (m = 1); q [rows, cols/8] FP32 or None (sigmoid = 1); s2 a one-element FP32
    device tensor, computed with ``tensor_scale`` when None."""
    _check_dev("w", w, torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    dev = w.device
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    if m is not None:
        _check_dev("m", m, torch.float32, dev)
        if tuple(m.shape) != (rows, cols // 16):
            raise ValueError(f"m must be [{rows}, {cols // 16}]")
    if q is not None:
        _check_dev("q", q, torch.float32, dev)
        if tuple(q.shape) != (rows, cols // 8):
            raise ValueError(f"q must be [{rows}, {cols // 8}]")
    if s2 is None:
        s2, _ = tensor_scale(w)
    _check_dev("s2", s2, torch.float32, dev)
    if s2.numel() < 1:
        raise ValueError("s2 must hold one float")
    codes, scales, deq, _ = _quant_outs(out, rows, cols, dev, dequant)
    _lib.check(_lib.lib().focus_quantize(_p(w), rows, cols, _p(m), _p(q), _p(s2), _p(codes),
                                         _p(scales), _p(deq), _stream(w)))
    return Quantized(codes, scales, deq, s2)


def dequantize(codes: torch.Tensor, scales: torch.Tensor, s2: torch.Tensor,
               s2_per_row: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """BF16 [rows, cols] = (c * S) * s2 from stored codes and scale bytes."""
    _check_dev("codes", codes, torch.uint8)
    dev = codes.device
    _check_dev("scales", scales, torch.uint8, dev)
    _check_dev("s2", s2, torch.float32, dev)
    rows, half = codes.shape
    cols = 2 * half
    if tuple(scales.shape) != (rows, cols // 16):
        raise ValueError(f"scales must be [{rows}, {cols // 16}]")
    if s2.numel() < (rows if s2_per_row else 1):
        raise ValueError("s2 too small")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _check_buf("out", out, torch.bfloat16, dev, rows * cols)
    _lib.check(_lib.lib().focus_dequantize(_p(codes), _p(scales), _p(s2), 1 if s2_per_row else 0,
                                           rows, cols, _p(out), _stream(codes)))
    return out


def quantize_act_per_token(x: torch.Tensor, dequant: bool = False,
                           out: Optional[Quantized] = None) -> Quantized:
    """Per-token NVFP4 of activations X [tokens, hidden] (one s2 per row)."""
    _check_dev("x", x, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, hidden]")
    t, h = x.shape
    if h % 16:
        raise ValueError("hidden must be a multiple of 16")
    dev = x.device
    codes, scales, deq, s2 = _quant_outs(out, t, h, dev, dequant, s2_rows=t)
    _lib.check(_lib.lib().focus_quantize_act_per_token(_p(x), t, h, _p(codes), _p(scales), _p(s2),
                                                       _p(deq), _stream(x)))
    return Quantized(codes, scales, deq, s2)


# ---------------------------------------------------------------------------
# FourOverSix
# ---------------------------------------------------------------------------

def quantize_fo6(w: torch.Tensor, s2: Optional[torch.Tensor] = None, dequant: bool = True,
                 out: Optional[Quantized] = None) -> Quantized:
    """FourOverSix round-to-nearest NVFP4 of W [rows, cols] (per-tensor s2,
    computed with ``tensor_scale`` when None)."""
    _check_dev("w", w, torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    dev = w.device
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    if s2 is None:
        s2, _ = tensor_scale(w)
    _check_dev("s2", s2, torch.float32, dev)
    if s2.numel() < 1:
        raise ValueError("s2 must hold one float")
    codes, scales, deq, _ = _quant_outs(out, rows, cols, dev, dequant)
    _lib.check(_lib.lib().focus_quantize_fo6(_p(w), rows, cols, _p(s2), _p(codes), _p(scales),
                                             _p(deq), _stream(w)))
    return Quantized(codes, scales, deq, s2)


def quantize_act_per_token_fo6(x: torch.Tensor, dequant: bool = False,
                               out: Optional[Quantized] = None) -> Quantized:
    """Per-token FourOverSix NVFP4 of activations X [tokens, hidden]."""
    _check_dev("x", x, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, hidden]")
    t, h = x.shape
    if h % 16:
        raise ValueError("hidden must be a multiple of 16")
    dev = x.device
    codes, scales, deq, s2 = _quant_outs(out, t, h, dev, dequant, s2_rows=t)
    _lib.check(_lib.lib().focus_quantize_act_per_token_fo6(_p(x), t, h, _p(codes), _p(scales),
                                                           _p(s2), _p(deq), _stream(x)))
    return Quantized(codes, scales, deq, s2)


# ---------------------------------------------------------------------------
# FOCUS on MXFP4
# ---------------------------------------------------------------------------

def _mx_outs(out, rows, cols, dev, dequant, label="out"):
    codes, scales, deq, _ = _quant_outs(out, rows, cols, dev, dequant, scale_block=32, label=label,
                                        deq_optional=label != "out")
    return Quantized(codes, scales, deq, None)


def quantize_mx(w: torch.Tensor, m: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                dequant: bool = True, out: Optional[Quantized] = None) -> Quantized:
    """FOCUS on MXFP4 of W [rows, cols] (cols % 32 == 0): m [rows, cols/32] or
    None, q [rows, cols/8] or None.  Returns codes, E8M0 scale bytes
    [rows, cols/32], optional BF16 w' (s2 is None: MXFP4 has no tensor scale)."""
    _check_dev("w", w, torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    dev = w.device
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    if m is not None:
        _check_dev("m", m, torch.float32, dev)
        if tuple(m.shape) != (rows, cols // 32):
            raise ValueError(f"m must be [{rows}, {cols // 32}]")
    if q is not None:
        _check_dev("q", q, torch.float32, dev)
        if tuple(q.shape) != (rows, cols // 8):
            raise ValueError(f"q must be [{rows}, {cols // 8}]")
    out = _mx_outs(out, rows, cols, dev, dequant)
    _lib.check(_lib.lib().focus_quantize_mx(_p(w), rows, cols, _p(m), _p(q), _p(out.codes),
                                            _p(out.scales), _p(out.deq), _stream(w)))
    return out


def dequantize_mx(codes: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _check_dev("codes", codes, torch.uint8)
    dev = codes.device
    _check_dev("scales", scales, torch.uint8, dev)
    rows, half = codes.shape
    cols = 2 * half
    if tuple(scales.shape) != (rows, cols // 32):
        raise ValueError(f"scales must be [{rows}, {cols // 32}]")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _check_buf("out", out, torch.bfloat16, dev, rows * cols)
    _lib.check(_lib.lib().focus_dequantize_mx(_p(codes), _p(scales), rows, cols, _p(out), _stream(codes)))
    return out


def quantize_mx_many(ws, ms, qs, outs=None, dequant: bool = True, run: bool = True) -> Batch:
    """Batched FOCUS on MXFP4 (m [rows, cols/32] entries may be None)."""
    n = len(ws)
    if not (len(ms) == len(qs) == n) or (outs is not None and len(outs) != n):
        raise ValueError("ws, ms, qs (and outs) must have the same length")
    if n == 0:
        raise ValueError("no tensors")
    dev = ws[0].device
    arr = (_lib.QuantDesc * n)()
    res = []
    for i in range(n):
        w, m, q = ws[i], ms[i], qs[i]
        _check_dev(f"ws[{i}]", w, torch.bfloat16, dev)
        if w.dim() != 2:
            raise ValueError(f"ws[{i}] must be 2-D [rows, cols]")
        rows, cols = w.shape
        if cols % 32:
            raise ValueError("cols must be a multiple of 32")
        if m is not None:
            _check_dev(f"ms[{i}]", m, torch.float32, dev)
            if tuple(m.shape) != (rows, cols // 32):
                raise ValueError(f"ms[{i}] must be [{rows}, {cols // 32}]")
        if q is not None:
            _check_dev(f"qs[{i}]", q, torch.float32, dev)
            if tuple(q.shape) != (rows, cols // 8):
                raise ValueError(f"qs[{i}] must be [{rows}, {cols // 8}]")
        o = _mx_outs(None if outs is None else outs[i], rows, cols, dev, dequant, label=f"outs[{i}]")
        res.append(o)
        arr[i] = _lib.QuantDesc(_p(w), rows, cols, _p(m), _p(q), 0, _p(o.codes), _p(o.scales), _p(o.deq))
    b = Batch("focus_quantize_mx_many", arr, (list(ws), list(ms), list(qs), res), dev)
    b.outs = res
    return b.run() if run else b


# ---------------------------------------------------------------------------
# FlipQuant MixFP4
# ---------------------------------------------------------------------------

def _mix_desc(i, w, tile_map, tile_rows, tile_cols, s2, dev, dequant, out):
    _check_dev(f"ws[{i}]", w, torch.bfloat16, dev)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    if tile_rows < 1 or tile_cols < 16 or tile_cols % 16 or rows % tile_rows or cols % tile_cols:
        raise ValueError("tiles must divide the tensor and tile_cols must be a multiple of 16")
    _check_dev(f"maps[{i}]", tile_map, torch.uint8, dev)
    if tuple(tile_map.shape) != (rows // tile_rows, cols // tile_cols) or not tile_map.is_contiguous():
        raise ValueError(f"map must be a contiguous [{rows // tile_rows}, {cols // tile_cols}] uint8 tensor")
    _check_dev(f"s2s[{i}]", s2, torch.float32, dev)
    if s2.numel() < 1:
        raise ValueError(f"s2s[{i}] must hold one float")
    codes, scales, deq, _ = _quant_outs(out, rows, cols, dev, dequant, label=f"outs[{i}]", deq_optional=True)
    res = Quantized(codes, scales, deq, s2)
    return res, _lib.MixDesc(_p(w), rows, cols, _p(s2), _p(tile_map), tile_rows, tile_cols, _p(codes),
                             _p(scales), _p(deq))


def quantize_mixfp4(w: torch.Tensor, tile_map: torch.Tensor, tile_rows: int, tile_cols: int = 64,
                    s2: Optional[torch.Tensor] = None, dequant: bool = True,
                    out: Optional[Quantized] = None) -> Quantized:
    """FlipQuant MixFP4 of W [rows, cols]: tile_map [rows/tile_rows,
    cols/tile_cols] uint8 (nonzero = E0M3 levels 0..7, zero = E2M1 with
    FourOverSix); per-tensor s2 computed with ``tensor_scale`` when None."""
    _check_dev("w", w, torch.bfloat16)
    if s2 is None:
        s2, _ = tensor_scale(w)
    res, d = _mix_desc(0, w, tile_map, tile_rows, tile_cols, s2, w.device, dequant, out)
    _lib.check(_lib.lib().focus_quantize_mixfp4(d.w_bf16, d.rows, d.cols, d.s2, d.map, d.tile_rows,
                                                d.tile_cols, d.codes, d.scales, d.w_deq, _stream(w)))
    return res


def quantize_mixfp4_many(ws, maps, tiles, s2s, outs=None, dequant: bool = True, run: bool = True) -> "Batch":
    """Batched MixFP4: maps[i] and tiles[i] = (tile_rows, tile_cols) per
    tensor; s2s one-element FP32 tensors; the result's ``outs`` holds the
    outputs."""
    n = len(ws)
    if not (len(maps) == len(tiles) == len(s2s) == n):
        raise ValueError("ws, maps, tiles, s2s must have the same length")
    dev = ws[0].device
    arr = (_lib.MixDesc * n)()
    res = []
    for i in range(n):
        r, arr[i] = _mix_desc(i, ws[i], maps[i], tiles[i][0], tiles[i][1], s2s[i], dev, dequant,
                              None if outs is None else outs[i])
        res.append(r)
    b = Batch("focus_quantize_mixfp4_many", arr, (list(ws), list(maps), list(s2s), res), dev)
    b.outs = res
    return b.run() if run else b


def dequantize_mixfp4(codes: torch.Tensor, scales: torch.Tensor, s2: torch.Tensor, tile_map: torch.Tensor,
                      tile_rows: int, tile_cols: int = 64, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stored MixFP4 codes [rows, cols/2] and scales [rows, cols/16] -> BF16
    [rows, cols]; tile_map as for ``quantize_mixfp4``."""
    dev = codes.device
    _check_dev("codes", codes, torch.uint8, dev)
    _check_dev("scales", scales, torch.uint8, dev)
    _check_dev("s2", s2, torch.float32, dev)
    _check_dev("tile_map", tile_map, torch.uint8, dev)
    rows, cols = codes.shape[0], 2 * codes.shape[1]
    if tuple(scales.shape) != (rows, cols // 16) or not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes [rows, cols/2] and scales [rows, cols/16] must be contiguous")
    if tuple(tile_map.shape) != (rows // max(tile_rows, 1), cols // max(tile_cols, 1)) or not tile_map.is_contiguous():
        raise ValueError("tile_map must be a contiguous [rows/tile_rows, cols/tile_cols] uint8 tensor")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _check_buf("out", out, torch.bfloat16, dev, rows * cols)
    _lib.check(_lib.lib().focus_dequantize_mixfp4(_p(codes), _p(scales), _p(s2), _p(tile_map), rows, cols, tile_rows,
                                                  tile_cols, _p(out), _stream(codes)))
    return out


# ---------------------------------------------------------------------------
# the NVFP4 linear layer
# ---------------------------------------------------------------------------

def nvfp4_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes for ``nvfp4_linear`` to split the sum over k (0: none)."""
    n = int(_lib.lib().focus_nvfp4_linear_workspace_bytes(M, N, K))
    if n < 0:
        raise FocusError(4, "the device query of the split model failed")
    return n


def nvfp4_linear(x: Quantized, w: Quantized, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Y = X' W'^T for NVFP4 activations ``x`` (codes [M, K/2], scales
    [M, K/16], s2 [M] per token or one value) and NVFP4 weights ``w`` (codes
    [N, K/2], scales [N, K/16], one s2), on the matrix cores; Y [M, N] in
    ``out_dtype`` (bfloat16 or float32).  ``workspace``: "auto" allocates the
    split-k workspace the library asks for, None uses none, or a float32
    device tensor."""
    dev = x.codes.device
    for name, t in (("x.codes", x.codes), ("x.scales", x.scales), ("w.codes", w.codes), ("w.scales", w.scales)):
        _check_dev(name, t, torch.uint8, dev)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _check_dev("x.s2", x.s2, torch.float32, dev)
    _check_dev("w.s2", w.s2, torch.float32, dev)
    M, K = x.codes.shape[0], 2 * x.codes.shape[1]
    N = w.codes.shape[0]
    if w.codes.shape[1] * 2 != K or tuple(x.scales.shape) != (M, K // 16) or tuple(w.scales.shape) != (N, K // 16):
        raise ValueError("operand shapes do not match: x [M, K], w [N, K] with K % 16 == 0")
    if x.s2.numel() not in (1, M) or w.s2.numel() != 1:
        raise ValueError("x.s2 needs 1 or M values, w.s2 one")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _check_dev("out", out, out_dtype, dev)
        if tuple(out.shape) != (M, N) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [M, N] tensor")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a float32 tensor")
        nbytes = nvfp4_linear_workspace_bytes(M, N, K) if M and N else 0
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=dev) if nbytes else None
    if workspace is not None:
        _check_dev("workspace", workspace, torch.float32, dev)
    per_row = 1 if (x.s2.numel() == M and M > 1) else 0
    _lib.check(_lib.lib().focus_nvfp4_linear(_p(x.codes), _p(x.scales), _p(x.s2), per_row, M, _p(w.codes),
                                             _p(w.scales), _p(w.s2), N, K, _p(out),
                                             0 if out_dtype == torch.float32 else 1, _p(workspace),
                                             0 if workspace is None else workspace.numel() * 4,
                                             _stream(x.codes)))
    return out


def nvfp4_linear_grouped(x: Quantized, ws, out_dtype: torch.dtype = torch.bfloat16, outs=None,
                         workspace="auto"):
    """``nvfp4_linear`` of one activation ``x`` through several weights ``ws``
    (a list of Quantized: codes [N_i, K/2], scales [N_i, K/16], one s2) that
    share it, e.g. a layer's q, k and v: with up to 128 tokens one launch per
    run of 8 weights.  Returns the list of outputs [M, N_i] (``outs`` may
    supply them).  ``workspace`` as for ``nvfp4_linear`` (used only with
    more than 128 tokens, for the largest member's split)."""
    dev = x.codes.device
    for name, t in (("x.codes", x.codes), ("x.scales", x.scales)):
        _check_dev(name, t, torch.uint8, dev)
    _check_dev("x.s2", x.s2, torch.float32, dev)
    M, K = x.codes.shape[0], 2 * x.codes.shape[1]
    if tuple(x.scales.shape) != (M, K // 16):
        raise ValueError("x.scales must be [M, K/16]")
    if x.s2.numel() not in (1, M):
        raise ValueError("x.s2 needs 1 or M values")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    n = len(ws)
    if outs is not None and len(outs) != n:
        raise ValueError("outs must have one tensor per weight")
    arr = (_lib.LinearWeight * max(n, 1))()
    res = []
    for i, w in enumerate(ws):
        _check_dev(f"ws[{i}].codes", w.codes, torch.uint8, dev)
        _check_dev(f"ws[{i}].scales", w.scales, torch.uint8, dev)
        _check_dev(f"ws[{i}].s2", w.s2, torch.float32, dev)
        N = w.codes.shape[0]
        if w.codes.shape[1] * 2 != K or tuple(w.scales.shape) != (N, K // 16) or w.s2.numel() != 1:
            raise ValueError(f"ws[{i}] must be codes [N, K/2], scales [N, K/16] and one s2")
        o = outs[i] if outs is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
        _check_buf(f"outs[{i}]", o, out_dtype, dev, M * N)
        res.append(o)
        arr[i] = _lib.LinearWeight(_p(w.codes), _p(w.scales), _p(w.s2), N, _p(o))
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a float32 tensor")
        nbytes = max([nvfp4_linear_workspace_bytes(M, w.codes.shape[0], K) for w in ws] + [0]) \
            if M > 128 and K else 0
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=dev) if nbytes else None
    if workspace is not None:
        _check_dev("workspace", workspace, torch.float32, dev)
    per_row = 1 if (x.s2.numel() == M and M > 1) else 0
    _lib.check(_lib.lib().focus_nvfp4_linear_grouped(_p(x.codes), _p(x.scales), _p(x.s2), per_row, M, K, arr, n,
                                                     0 if out_dtype == torch.float32 else 1, _p(workspace),
                                                     0 if workspace is None else workspace.numel() * 4,
                                                     _stream(x.codes)))
    return res


def nvfp4_linear_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch that ``nvfp4_linear_noalloc`` uses."""
    return int(_lib.lib().focus_nvfp4_linear_scratch_bytes())


def nvfp4_linear_noalloc(x: Quantized, w: Quantized, out: torch.Tensor) -> torch.Tensor:
    """``nvfp4_linear`` into the caller's ``out`` ([M, N] bfloat16 or float32,
    contiguous) with the library's per-GPU scratch as the split-k workspace:
    neither this call nor the library allocates anything (usable under HIP
    graph capture).  Calls that may overlap on one GPU share that scratch and
    must be serialized by the caller."""
    dev = x.codes.device
    for name, t in (("x.codes", x.codes), ("x.scales", x.scales), ("w.codes", w.codes), ("w.scales", w.scales)):
        _check_dev(name, t, torch.uint8, dev)
    _check_dev("x.s2", x.s2, torch.float32, dev)
    _check_dev("w.s2", w.s2, torch.float32, dev)
    M, K = x.codes.shape[0], 2 * x.codes.shape[1]
    N = w.codes.shape[0]
    if w.codes.shape[1] * 2 != K or tuple(x.scales.shape) != (M, K // 16) or tuple(w.scales.shape) != (N, K // 16):
        raise ValueError("operand shapes do not match: x [M, K], w [N, K] with K % 16 == 0")
    if x.s2.numel() not in (1, M) or w.s2.numel() != 1:
        raise ValueError("x.s2 needs 1 or M values, w.s2 one")
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be a bfloat16 or float32 tensor")
    _check_buf("out", out, out.dtype, dev, M * N)
    per_row = 1 if (x.s2.numel() == M and M > 1) else 0
    _lib.check(_lib.lib().focus_nvfp4_linear_noalloc(_p(x.codes), _p(x.scales), _p(x.s2), per_row, M, _p(w.codes),
                                                     _p(w.scales), _p(w.s2), N, K, _p(out),
                                                     0 if out.dtype == torch.float32 else 1, _stream(x.codes)))
    return out


# ---------------------------------------------------------------------------
# batched calls
# ---------------------------------------------------------------------------

class Batch:
    """A prepared batched call: the descriptor array is built once (device
    pointers of the given tensors, which must stay alive), and ``run()``
    launches it on the current stream of ``device``."""

    def __init__(self, fn_name: str, descs, keep, device):
        self._fn = getattr(_lib.lib(), fn_name)
        self._descs = descs
        self._n = len(descs)
        self._keep = keep  # keep the tensors alive while the batch exists
        self.device = device

    def run(self):
        if self._n:
            _lib.check(self._fn(self._descs, self._n, torch.cuda.current_stream(self.device).cuda_stream))
        return self

    __call__ = run


def tensor_scale_many(ws, s2_out=None, amax_out=None, run: bool = True) -> Batch:
    """Tensor scales of several BF16 tensors.  s2_out / amax_out: FP32 tensors
    with one element per input (e.g. an [n, 1] tensor), allocated if None."""
    n = len(ws)
    if n == 0:
        raise ValueError("no tensors")
    dev = ws[0].device
    for i, w in enumerate(ws):
        _check_dev(f"ws[{i}]", w, torch.bfloat16, dev)
    if s2_out is None:
        s2_out = torch.empty((n, 1), dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty((n, 1), dtype=torch.float32, device=dev)
    _check_dev("s2_out", s2_out, torch.float32, dev)
    _check_dev("amax_out", amax_out, torch.float32, dev)
    if s2_out.numel() < n or amax_out.numel() < n:
        raise ValueError("s2_out / amax_out need one element per tensor")
    arr = (_lib.ScaleDesc * n)()
    s2f, amf = s2_out.view(-1), amax_out.view(-1)
    for i, w in enumerate(ws):
        arr[i] = _lib.ScaleDesc(_p(w), w.numel(), s2f[i].data_ptr(), amf[i].data_ptr())
    b = Batch("focus_tensor_scale_many", arr, (list(ws), s2_out, amax_out), dev)
    b.s2, b.amax = s2_out, amax_out
    return b.run() if run else b


def quantize_fo6_many(ws, s2s, outs=None, dequant: bool = True, run: bool = True) -> Batch:
    """Batched FourOverSix of several weight tensors (see ``quantize_many``)."""
    b = quantize_many(ws, [None] * len(ws), [None] * len(ws), s2s, outs=outs, dequant=dequant, run=False)
    b._fn = _lib.lib().focus_quantize_fo6_many
    return b.run() if run else b


def quantize_many(ws, ms, qs, s2s, outs=None, dequant: bool = True, run: bool = True) -> Batch:
    """FOCUS quantizer over several linears in as few launches as possible.
    ms / qs: lists (entries may be None); s2s: one-element FP32 tensors (for
    example the rows of ``tensor_scale_many(...).s2``); outs: list of
    ``Quantized`` output buffers, allocated if None.  The result's ``outs``
    holds the outputs."""
    n = len(ws)
    if not (len(ms) == len(qs) == len(s2s) == n):
        raise ValueError("ws, ms, qs, s2s must have the same length")
    if outs is not None and len(outs) != n:
        raise ValueError("outs must have one entry per tensor")
    if n == 0:
        raise ValueError("no tensors")
    dev = ws[0].device
    arr = (_lib.QuantDesc * n)()
    res = []
    for i in range(n):
        w, m, q, s2 = ws[i], ms[i], qs[i], s2s[i]
        _check_dev(f"ws[{i}]", w, torch.bfloat16, dev)
        if w.dim() != 2:
            raise ValueError(f"ws[{i}] must be 2-D [rows, cols]")
        rows, cols = w.shape
        if cols % 16:
            raise ValueError(f"ws[{i}]: cols must be a multiple of 16")
        if m is not None:
            _check_dev(f"ms[{i}]", m, torch.float32, dev)
            if tuple(m.shape) != (rows, cols // 16):
                raise ValueError(f"ms[{i}] must be [{rows}, {cols // 16}]")
        if q is not None:
            _check_dev(f"qs[{i}]", q, torch.float32, dev)
            if tuple(q.shape) != (rows, cols // 8):
                raise ValueError(f"qs[{i}] must be [{rows}, {cols // 8}]")
        _check_dev(f"s2s[{i}]", s2, torch.float32, dev)
        if s2.numel() < 1:
            raise ValueError(f"s2s[{i}] must hold one float")
        codes, scales, deq, _ = _quant_outs(None if outs is None else outs[i], rows, cols, dev, dequant,
                                            label=f"outs[{i}]", deq_optional=True)
        res.append(Quantized(codes, scales, deq, s2))
        arr[i] = _lib.QuantDesc(_p(w), rows, cols, _p(m), _p(q), _p(s2), _p(codes), _p(scales), _p(deq))
    b = Batch("focus_quantize_many", arr, (list(ws), list(ms), list(qs), list(s2s), res), dev)
    b.outs = res
    return b.run() if run else b


def dequantize_many(codes, scales, s2s, outs=None, s2_per_row=None, run: bool = True) -> Batch:
    """Dequantize several stored tensors; the result's ``outs`` holds them."""
    n = len(codes)
    if len(scales) != n or len(s2s) != n or (outs is not None and len(outs) != n) or \
            (s2_per_row is not None and len(s2_per_row) != n):
        raise ValueError("codes, scales, s2s (and outs, s2_per_row) must have the same length")
    if n == 0:
        raise ValueError("no tensors")
    dev = codes[0].device
    arr = (_lib.DequantDesc * n)()
    res = []
    for i in range(n):
        c, s, s2 = codes[i], scales[i], s2s[i]
        _check_dev(f"codes[{i}]", c, torch.uint8, dev)
        _check_dev(f"scales[{i}]", s, torch.uint8, dev)
        _check_dev(f"s2s[{i}]", s2, torch.float32, dev)
        if c.dim() != 2:
            raise ValueError(f"codes[{i}] must be 2-D [rows, cols/2]")
        rows, half = c.shape
        cols = 2 * half
        if cols % 16:
            raise ValueError(f"codes[{i}]: cols must be a multiple of 16")
        if s.numel() != rows * cols // 16:
            raise ValueError(f"scales[{i}] must hold [{rows}, {cols // 16}] bytes")
        pr = bool(s2_per_row[i]) if s2_per_row is not None else False
        if s2.numel() < (rows if pr else 1):
            raise ValueError(f"s2s[{i}] too small")
        o = outs[i] if outs is not None else torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
        _check_buf(f"outs[{i}]", o, torch.bfloat16, dev, rows * cols)
        res.append(o)
        arr[i] = _lib.DequantDesc(_p(c), _p(s), _p(s2), 1 if pr else 0, rows, cols, _p(o))
    b = Batch("focus_dequantize_many", arr, (list(codes), list(scales), list(s2s), res), dev)
    b.outs = res
    return b.run() if run else b
