"""Parity rule between the HIP path and the oracle, shared by the GPU tests
and the benchmark's check of every output of the 1B and 8B weight sets.

The bar:
  * scale bytes and s2 bit-exact;
  * E2M1 codes: at most floor(1e-6 * n) elements may differ, each by exactly
    one magnitude step, and only where re-running the oracle's element code
    with sigmoid moved by at most 2 binary32 ulps reproduces the GPU code
    (the one operation whose last-bit rounding may legitimately differ is
    expf inside sigmoid);
  * w' bit-exact wherever the codes agree.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CODE_MISMATCH_RATE = 1e-6


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def unpack(packed: np.ndarray) -> np.ndarray:
    return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[0], -1)


def oracle_quantize_rows(o, wb, m, q, s2, dequant=True, n_threads=None):
    """Oracle quantizer over row chunks on several threads (ctypes releases
    the GIL); the arithmetic per row is unchanged."""
    rows = wb.shape[0]
    n = n_threads or threads()
    if rows < 2 * n:
        return o.quantize(wb, m, q, s2, dequant)
    bounds = np.linspace(0, rows, n + 1).astype(int)

    def run(i):
        a, b = bounds[i], bounds[i + 1]
        return o.quantize(wb[a:b], None if m is None else m[a:b], None if q is None else q[a:b],
                          s2, dequant)

    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(run, range(n)))
    codes = np.concatenate([p[0] for p in parts])
    scales = np.concatenate([p[1] for p in parts])
    deq = np.concatenate([p[2] for p in parts]) if dequant else None
    return codes, scales, deq


def oracle_act_rows(o, xb, dequant=False, n_threads=None):
    rows = xb.shape[0]
    n = n_threads or threads()
    if rows < 2 * n:
        return o.quantize_act_per_token(xb, dequant)
    bounds = np.linspace(0, rows, n + 1).astype(int)
    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda i: o.quantize_act_per_token(xb[bounds[i]:bounds[i + 1]], dequant),
                            range(n)))
    out = [np.concatenate([p[k] for p in parts]) for k in range(3)]
    out.append(np.concatenate([p[3] for p in parts]) if dequant else None)
    return tuple(out)


def check_quantized(o, wb, m, q, s2, gpu_codes, gpu_scales, gpu_deq, ref=None, label="",
                    count_limit=None):
    """Compare GPU outputs (numpy, same rows as wb) with the oracle on the
    same inputs.  Returns a dict of counts; raises AssertionError when the
    parity bar fails.  ``count_limit`` replaces the 1e-6 bound on the number
    of code mismatches (a caller checking a tensor in parts applies the bound
    to the whole); every mismatch must still be one step explained by sigmoid
    rounding."""
    if ref is None:
        ref = oracle_quantize_rows(o, wb, m, q, s2, dequant=gpu_deq is not None)
    codes, scales, deq = ref
    assert gpu_scales.shape == scales.shape and gpu_codes.shape == codes.shape, label
    bad_s = np.count_nonzero(gpu_scales != scales)
    assert bad_s == 0, f"{label}: {bad_s} scale bytes differ, first at " \
                       f"{np.argwhere(gpu_scales != scales)[:4].tolist()}"
    gc, oc = unpack(gpu_codes), unpack(codes)
    diff = np.argwhere(gc != oc)
    n = gc.size
    allowed = int(np.floor(CODE_MISMATCH_RATE * n)) if count_limit is None else int(count_limit)
    assert len(diff) <= allowed, f"{label}: {len(diff)} code mismatches > {allowed} allowed of {n}; " \
                                 f"first {diff[:4].tolist()}"
    for r, c in diff:
        g, w = int(gc[r, c]), int(oc[r, c])
        assert (g & 8) == (w & 8) and abs((g & 7) - (w & 7)) == 1, f"{label}: not one step at {(r, c)}"
        assert q is not None, f"{label}: code mismatch without a sigmoid at {(r, c)}"
        S = o.e4m3_value(int(scales[r, c // 16]))
        sig = np.float32(o.sigmoid(float(q[r, c // 8])))
        ok = False
        for k in (-2, -1, 1, 2):
            s = sig
            for _ in range(abs(k)):
                s = np.nextafter(s, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            if o.element_code(int(wb[r, c]), S, float(s), float(s2)) == g:
                ok = True
                break
        assert ok, f"{label}: code mismatch at {(r, c)} not explained by sigmoid rounding"
    if gpu_deq is not None:
        agree = (gc == oc)
        bad_d = np.count_nonzero((gpu_deq != deq) & agree)
        assert bad_d == 0, f"{label}: {bad_d} w' values differ where codes agree, first at " \
                           f"{np.argwhere((gpu_deq != deq) & agree)[:4].tolist()}"
    return {"elements": n, "code_mismatches": len(diff), "allowed": allowed}
