"""Benchmark of the FOCUS NVFP4 quantizer on one MI355X.

One step is one pass of the whole path over the Llama-3.1-8B-shaped weight
set (224 linears, 6,979,321,856 weights) plus one batch of activations:

  1. focus_tensor_scale     for every linear (s2 = amax|W| / 2688)
  2. focus_quantize         for every linear, codes + scale bytes + fused w'
  3. focus_dequantize       for every linear (codes + scales -> BF16)
  4. focus_quantize_act_per_token on X [8192, 4096]

Phases run in this order so that each kernel streams its operands from HBM
(the set is 23 GB, far beyond the 256 MB last-level cache).  Inputs are
generated on the GPU before the timed region (seeded, synthetic; see
``synth``) and stay resident in HBM.

``value`` is whole-step throughput in Gweights/s (weights of the set per
second of step time); ``quantize_gweights_s`` is the quantize + w' phase
alone (the quantize+pack figure), ``quantize_codes_only_gweights_s`` the
quantizer without w'.  ``roofline`` reports the dominant kernel,
focus_quantize with w', against the 8 TB/s HBM peak: algorithmic bytes
(5.3125 B per weight) / mean launch duration, every launch bracketed by HIP
events on the stream it runs on, and against a hand-written streaming
kernel that moves one launch's read and write bytes in the same process.
``rows`` breaks the step down per call and adds rows timed after the steps:
codes-only quantize, the adjacent formats (FourOverSix also with its weights
served from the last-level cache, which isolates its arithmetic),
traffic-pattern ceilings of the quantizer, the tensor scale, the dequantize
and the activations (back to back, and for the activations also in the
activation phase's position in the step), the linear layer (8192, 2048 and 16 tokens; one decoder layer as a
HIP graph replay, and eight distinct layers whose weights stream from HBM),
and the Llama-3.2-1B-shaped set's step.

``parity``: right after the timed steps, every output of the last step
(s2, amax, scale bytes, codes, w' and the dequantized copy of all 224
linears, and the per-token activations) is compared with the CPU oracle run
on the same input bytes; ``parity_1b`` does the same for the 1B set.  The
oracle's timed quantize passes over the whole set are ``cpu_baseline``.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b|1b|70b]
                       [--no-parity] [--no-1b]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gweights/s + achieved HBM GB/s (% of peak), FOCUS NVFP4 quantize+pack, 8B set"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense FP16 matrix-core peak (the linear layer's contraction type)

# algorithmic bytes per weight (per element for activations)
B_TENSOR_SCALE = 2.0
B_QUANT = 2.0 + 0.25 + 0.5 + 0.5 + 0.0625          # W, m, q, codes, scales
B_QUANT_DQ = B_QUANT + 2.0                          # + w'
B_DEQUANT = 0.5 + 0.0625 + 2.0                      # codes, scales, out
B_ACT = 2.0 + 0.5 + 0.0625                          # X, codes, scales (+4 B per token)
B_MX = 2.0 + 4.0 / 32 + 0.5 + 0.5 + 1.0 / 32        # W, m per 32, q, codes, E8M0 scales

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "quantize_8b_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["8b", "1b", "70b"], default="8b",
                    help="8b (default): the Llama-3.1-8B-shaped set; 1b: Llama-3.2-1B-shaped; "
                         "70b: Llama-3.1-70B-shaped, processed layer by layer with w' and the "
                         "dequantized copy written to one reused per-layer buffer")
    ap.add_argument("--no-parity", "--no-cpu-baseline", dest="no_parity", action="store_true",
                    help="skip the oracle pass (parity of every output and the CPU baseline), e.g. "
                         "for profiled runs")
    ap.add_argument("--no-1b", action="store_true",
                    help="skip the Llama-3.2-1B-shaped set's step row (8b workload)")
    ap.add_argument("--cpu-weights", type=float, default=0,
                    help="stop the oracle pass after this many weights (0: the whole set)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the steps, copy a buffer of BYTES bytes three times (a plain copy "
                         "kernel of known traffic, to scale hardware byte counters)")
    return ap.parse_args()


# The sources the quantize kernel is compiled from.
QUANT_KERNEL_SOURCES = ("focus_internal.h", "focus_kernels.hip", "focus_numerics.h")


def kernel_source_hash() -> str:
    """Hash of the quantize kernel's code: its sources with comments and
    whitespace removed, so only a change to the code itself invalidates a
    stored measurement."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_post_weight_amd", "csrc")
    for name in QUANT_KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = "".join(code.split())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """Per-launch HBM traffic of the dominant kernel from the committed
    rocprofv3 counter summary, or None when it is absent or was taken on
    other kernel sources."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


class WeightSetRun:
    """One weight set resident in HBM with its outputs and the prepared
    batched calls of a step: tensor scale, quantize with w', dequantize (one
    launch per run of up to 32 linears; per layer for the layered 70B set,
    whose w' and dequantized copy go to one reused per-layer buffer)."""

    def __init__(self, focus, synth, ws, dev, layered=False):
        import torch
        self.ws, self.layered = ws, layered
        self.lins = ws.linears()
        self.n_weights = sum(l.numel for l in self.lins)
        lins = self.lins
        self.W, self.M, self.Q = [], [], []
        for lin in lins:
            w, m, q = synth.make_linear(ws, lin, device=dev)
            self.W.append(w)
            self.M.append(m)
            self.Q.append(q)
        n = len(lins)
        self.S2 = torch.empty((n, 1), dtype=torch.float32, device=dev)
        self.AMAX = torch.empty((n, 1), dtype=torch.float32, device=dev)
        if layered:
            per_layer = max(sum(l.numel for l in lins if l.layer == k) for k in range(ws.layers))
            wdq_buf = torch.empty(per_layer, dtype=torch.bfloat16, device=dev)
            deq_buf = torch.empty(per_layer, dtype=torch.bfloat16, device=dev)
            self.WDQ, self.DEQ, off = [], [], {}
            for l in lins:
                o = off.get(l.layer, 0)
                self.WDQ.append(wdq_buf[o:o + l.numel].view(l.rows, l.cols))
                self.DEQ.append(deq_buf[o:o + l.numel].view(l.rows, l.cols))
                off[l.layer] = o + l.numel
            self.chunks = [[i for i, l in enumerate(lins) if l.layer == k] for k in range(ws.layers)]
        else:
            self.WDQ = [torch.empty((l.rows, l.cols), dtype=torch.bfloat16, device=dev) for l in lins]
            self.DEQ = [torch.empty((l.rows, l.cols), dtype=torch.bfloat16, device=dev) for l in lins]
            self.chunks = [list(range(i, min(i + 32, n))) for i in range(0, n, 32)]
        self.OUT = [focus.Quantized(torch.empty((l.rows, l.cols // 2), dtype=torch.uint8, device=dev),
                                    torch.empty((l.rows, l.cols // 16), dtype=torch.uint8, device=dev),
                                    self.WDQ[i], self.S2[i]) for i, l in enumerate(lins)]
        c_ = self.chunks
        W, M, Q, S2, OUT = self.W, self.M, self.Q, self.S2, self.OUT
        self.TS = [focus.tensor_scale_many([W[i] for i in c], S2[c[0]:c[-1] + 1], self.AMAX[c[0]:c[-1] + 1],
                                           run=False) for c in c_]
        self.QB = [focus.quantize_many([W[i] for i in c], [M[i] for i in c], [Q[i] for i in c],
                                       [S2[i] for i in c], outs=[OUT[i] for i in c], dequant=True, run=False)
                   for c in c_]
        self.QB_nodq = [focus.quantize_many([W[i] for i in c], [M[i] for i in c], [Q[i] for i in c],
                                            [S2[i] for i in c], outs=[OUT[i] for i in c], dequant=False,
                                            run=False) for c in c_]
        self.DB = [focus.dequantize_many([OUT[i].codes for i in c], [OUT[i].scales for i in c],
                                         [S2[i] for i in c], outs=[self.DEQ[i] for i in c], run=False)
                   for c in c_]

    def step(self, rec=None, q_rec=None):
        """tensor scale -> quantize + w' -> dequantize of every linear;
        rec(k) records phase boundary k (0: start, 1: scales done, 2:
        quantize done, 3: dequantize done); q_rec(i, 0/1) brackets quantize
        launch i."""
        rec = rec or (lambda k: None)
        rec(0)
        for b in self.TS:
            b.run()
        rec(1)
        for i, b in enumerate(self.QB):
            if q_rec:
                q_rec(i, 0)
            b.run()
            if q_rec:
                q_rec(i, 1)
        rec(2)
        for b in self.DB:
            b.run()
        rec(3)


def _stream_lib():
    import ctypes as ct
    lib = ct.CDLL(os.path.join(ROOT, "tests", "hip", "libfocus_stream.so"))
    lib.focus_stream_pattern.restype = ct.c_int
    lib.focus_stream_pattern.argtypes = [ct.c_void_p] * 3 + [ct.c_int64] + [ct.c_void_p] * 3 + [ct.c_int, ct.c_void_p]
    lib.focus_stream_act_pattern.restype = ct.c_int
    lib.focus_stream_act_pattern.argtypes = [ct.c_void_p, ct.c_int64, ct.c_int] + [ct.c_void_p] * 3 + \
        [ct.c_int64, ct.c_void_p]
    lib.focus_stream_read_pattern.restype = ct.c_int
    lib.focus_stream_read_pattern.argtypes = [ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_int, ct.c_int64, ct.c_void_p]
    lib.focus_stream_deq_pattern.restype = ct.c_int
    lib.focus_stream_deq_pattern.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_int64, ct.c_void_p, ct.c_void_p]
    return lib


def _time_stream(fn, reps=5):
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def stream_ceiling(dev, nblk, reps=5):
    """The hand-written kernel of tests/hip/focus_stream.hip: the memory
    traffic of one quantize + w' launch over `nblk` 16-element blocks (W, m
    and q in; codes, scales and w' out, 85 bytes per block) with the
    quantizer's work layout and no arithmetic, at 1, 2 and 4 blocks per lane,
    timed with HIP events; the fastest.  Returns (ms, GB/s, blocks per lane)."""
    import torch
    lib = _stream_lib()
    w = torch.ones(nblk * 16, dtype=torch.bfloat16, device=dev)
    m = torch.ones(nblk, dtype=torch.float32, device=dev)
    q = torch.ones(nblk * 2, dtype=torch.float32, device=dev)
    codes = torch.empty(nblk * 8, dtype=torch.uint8, device=dev)
    scales = torch.empty(nblk, dtype=torch.uint8, device=dev)
    wdeq = torch.empty_like(w)
    stream = torch.cuda.current_stream(dev)
    best = None
    for u in (1, 2, 4):
        def call(u=u):
            st = lib.focus_stream_pattern(w.data_ptr(), m.data_ptr(), q.data_ptr(), nblk, codes.data_ptr(),
                                          scales.data_ptr(), wdeq.data_ptr(), u, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"focus_stream_pattern failed with HIP error {st}")
        ms = _time_stream(call, reps)
        if best is None or ms < best[0]:
            best = (ms, u)
    del w, m, q, codes, scales, wdeq
    return best[0], nblk * 85.0 / (best[0] * 1e-3) / 1e9, best[1]


def act_ceiling(dev, tokens, hidden, reps=20):
    """The activation kernel's traffic (X [tokens, hidden] in; codes, scale
    bytes and one float per token out) with its work layout (a wavefront per
    row, rows taken in turn, two per wavefront, at least 1024 workgroups) and
    no arithmetic.  Returns (ms, GB/s)."""
    import torch
    lib = _stream_lib()
    rb = hidden // 1024
    x = torch.ones((tokens, hidden), dtype=torch.bfloat16, device=dev)
    codes = torch.empty(tokens * hidden // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(tokens * hidden // 16, dtype=torch.uint8, device=dev)
    s2 = torch.empty(tokens, dtype=torch.float32, device=dev)
    g1 = (tokens + 3) // 4
    g = (tokens + 7) // 8
    if g < 1024:
        g = g1 if g1 < 1024 else 1024
    stream = torch.cuda.current_stream(dev)

    def call():
        st = lib.focus_stream_act_pattern(x.data_ptr(), tokens, rb, codes.data_ptr(), scales.data_ptr(), s2.data_ptr(),
                                          g, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"focus_stream_act_pattern failed with HIP error {st}")
    ms = _time_stream(call, reps)
    nbytes = B_ACT * tokens * hidden + 4 * tokens
    del x, codes, scales, s2
    return ms, nbytes / (ms * 1e-3) / 1e9


def read_ceiling(dev, nvec, reps=5):
    """The tensor scale's traffic (nvec 16-byte vectors read once, nothing
    written but one word per lane) with its work layout (256-lane workgroups
    striding over tiles, u nontemporal 16-byte loads per lane per tile) and no
    arithmetic, at u = 4 or 8 and 1024, 2048 or 8192 workgroups; the fastest.
    Returns (ms, GB/s, u, workgroups)."""
    import torch
    lib = _stream_lib()
    w = torch.ones(nvec * 8, dtype=torch.bfloat16, device=dev)
    out = torch.empty(8192 * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for u in (4, 8):
        for g in (1024, 2048, 8192):
            def call(u=u, g=g):
                st = lib.focus_stream_read_pattern(w.data_ptr(), nvec, out.data_ptr(), u, g, stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"focus_stream_read_pattern failed with HIP error {st}")
            ms = _time_stream(call, reps)
            if best is None or ms < best[0]:
                best = (ms, u, g)
    del w, out
    return best[0], nvec * 16.0 / (best[0] * 1e-3) / 1e9, best[1], best[2]


def deq_ceiling(dev, nblk, reps=5):
    """The dequantize's traffic (codes and a scale byte per 16-element block
    in, 32 bytes of BF16 out) with its work layout (one block per lane per
    tile, output regrouped through LDS into 1 KB contiguous nontemporal
    stores) and no arithmetic.  Returns (ms, GB/s)."""
    import torch
    lib = _stream_lib()
    codes = torch.ones(nblk * 8, dtype=torch.uint8, device=dev)
    scales = torch.ones(nblk, dtype=torch.uint8, device=dev)
    out = torch.empty(nblk * 32, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        st = lib.focus_stream_deq_pattern(codes.data_ptr(), scales.data_ptr(), nblk, out.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"focus_stream_deq_pattern failed with HIP error {st}")
    ms = _time_stream(call, reps)
    del codes, scales, out
    return ms, nblk * 41.0 / (ms * 1e-3) / 1e9


def act_step_position(focus, R, X, ACT, dev, reps=6):
    """Mean time of the activation phase in the step's position (tensor scale,
    quantize and dequantize of the set run first, so X is not in the caches),
    for the quantizer and for the no-arithmetic kernel with its traffic and
    work layout writing the same buffers, alternated.  Returns (ms, ms)."""
    import torch
    lib = _stream_lib()
    tokens, hidden = X.shape
    g1 = (tokens + 3) // 4
    g = (tokens + 7) // 8
    if g < 1024:
        g = g1 if g1 < 1024 else 1024
    stream = torch.cuda.current_stream(dev)

    def pattern():
        st = lib.focus_stream_act_pattern(X.data_ptr(), tokens, hidden // 1024, ACT.codes.data_ptr(),
                                          ACT.scales.data_ptr(), ACT.s2.data_ptr(), g, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"focus_stream_act_pattern failed with HIP error {st}")

    calls = (lambda: focus.quantize_act_per_token(X, out=ACT), pattern)
    tot = [0.0, 0.0]
    for r in range(reps):
        for i, fn in enumerate(calls):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            R.step()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            tot[i] += a.elapsed_time(b)
    return tot[0] / reps, tot[1] / reps


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the quantizer is measured on one MI355X "
              "(multi-GPU sharding is a design note only). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_post_weight_amd as focus
    import synth

    focus._lib.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = {"8b": synth.LLAMA_8B, "1b": synth.LLAMA_1B, "70b": synth.LLAMA_70B}[args.workload]
    layered = args.workload == "70b"

    # ---- inputs (resident in HBM) and outputs ----------------------------
    t0 = time.time()
    R = WeightSetRun(focus, synth, ws, dev, layered)
    lins, n_weights, nlin = R.lins, R.n_weights, len(R.lins)
    W, M, Q, S2, OUT = R.W, R.M, R.Q, R.S2, R.OUT
    X = synth.make_activations(device=dev)
    ACT = focus.quantize_act_per_token(X)
    torch.cuda.synchronize()
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"generated {ws.name}: {n_weights} weights in {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream(dev)
    nq = len(R.QB)

    # events of one step: [0] start, [1] tensor scales done, a pair around
    # each quantize launch, quantize phase done, dequantize done, act done
    n_ev = 5 + 2 * nq
    E_TS, E_Q0, E_QEND, E_DQ, E_ACT = 1, 2, 2 + 2 * nq, 3 + 2 * nq, 4 + 2 * nq

    def step(ev=None):
        if ev is None:
            R.step()
        else:
            pos = {0: 0, 1: E_TS, 2: E_QEND, 3: E_DQ}
            R.step(lambda k: ev[pos[k]].record(stream), lambda i, e: ev[E_Q0 + 2 * i + e].record(stream))
        focus.quantize_act_per_token(X, out=ACT)
        if ev is not None:
            ev[E_ACT].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region -------------------------------------------------------
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    gpu_ms = events[0][0].elapsed_time(events[-1][E_ACT])
    ms_step = max(gpu_ms, wall * 1e3) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms per step")

    q_launch_ms = []
    phase = {"tensor_scale": 0.0, "quantize_dq": 0.0, "dequantize": 0.0, "act": 0.0}
    for k in range(args.steps):
        ev = events[k]
        for i in range(nq):
            q_launch_ms.append(ev[E_Q0 + 2 * i].elapsed_time(ev[E_Q0 + 2 * i + 1]))
        phase["tensor_scale"] += ev[0].elapsed_time(ev[E_TS])
        phase["quantize_dq"] += ev[E_TS].elapsed_time(ev[E_QEND])
        phase["dequantize"] += ev[E_QEND].elapsed_time(ev[E_DQ])
        phase["act"] += ev[E_DQ].elapsed_time(ev[E_ACT])
    phase = {k: v / args.steps for k, v in phase.items()}
    mean_launch_ms = float(np.mean(q_launch_ms))
    bytes_per_launch = B_QUANT_DQ * n_weights / nq
    achieved = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9

    # ---- parity of every output of the timed steps against the oracle -----
    # (before any later row overwrites the output buffers); its oracle pass
    # is also the CPU baseline
    par, cpu = None, None
    if not args.no_parity:
        par, cpu = check_set(R, X, ACT, args, layered, label=args.workload.upper())
        for _ in range(2):  # the GPU idled during the oracle pass
            step()
        torch.cuda.synchronize()

    # ---- per-call rows outside the steps: each call alone, same buffers ----
    def time_calls(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def row(ms, nbytes, units):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "Gunits_s": round(units / (ms * 1e-3) / 1e9, 2)}

    t_q = time_calls(lambda: [b.run() for b in R.QB_nodq])
    rows = {
        "tensor_scale (step phase)": row(phase["tensor_scale"], B_TENSOR_SCALE * n_weights, n_weights),
        "quantize + w' (step phase)": row(phase["quantize_dq"], B_QUANT_DQ * n_weights, n_weights),
        "dequantize (step phase)": row(phase["dequantize"], B_DEQUANT * n_weights, n_weights),
        "act per token [8192,4096] (step phase)": row(phase["act"], B_ACT * X.numel() + 4 * X.shape[0],
                                                      X.numel()),
        "quantize codes only (after the steps)": row(t_q, B_QUANT * n_weights, n_weights),
    }
    extra_rows = not layered
    if extra_rows:
        chunks = R.chunks
        FB = [focus.quantize_fo6_many([W[i] for i in c], [S2[i] for i in c], outs=[OUT[i] for i in c],
                                      dequant=False, run=False) for c in chunks]
        M32 = [synth.block_factor_lognormal((l.rows, l.cols // 32), seed=42, tensor_id=l.tid(1), device=dev)
               for l in lins]

        def mx_out(i, dq):
            sc = OUT[i].scales.view(-1)[:lins[i].numel // 32].view(lins[i].rows, lins[i].cols // 32)
            return focus.Quantized(OUT[i].codes, sc, OUT[i].deq if dq else None, None)

        MXB = [focus.quantize_mx_many([W[i] for i in c], [M32[i] for i in c], [Q[i] for i in c],
                                      outs=[mx_out(i, True) for i in c], dequant=True, run=False) for c in chunks]
        MXB_nodq = [focus.quantize_mx_many([W[i] for i in c], [M32[i] for i in c], [Q[i] for i in c],
                                           outs=[mx_out(i, False) for i in c], dequant=False, run=False)
                    for c in chunks]
        MIX_TILES = [(8, 64), (16, 64), (256, 64)]
        MAPS = {t: [synth.tile_map(l.rows, l.cols, t, frac=synth.MIXFP4_FRAC[t], seed=42, tensor_id=l.tid(3),
                                   device=dev) for l in lins] for t in MIX_TILES}
        MIXB = {t: [focus.quantize_mixfp4_many([W[i] for i in c], [MAPS[t][i] for i in c], [t] * len(c),
                                               [S2[i] for i in c], outs=[OUT[i] for i in c], dequant=True,
                                               run=False) for c in chunks] for t in MIX_TILES}
        t_f6 = time_calls(lambda: [b.run() for b in FB])
        # The same FourOverSix launches (same shapes, batches and outputs) with
        # every linear reading the set's largest tensor (117 MB, so after the
        # first touch its bytes come from the 256 MB last-level cache, not
        # HBM): if the time does not drop, the kernel's rate is set by its
        # arithmetic, not by its weight reads.
        src = max(range(nlin), key=lambda i: lins[i].numel)
        wsrc = W[src].view(-1)
        FBc = [focus.quantize_fo6_many([wsrc[:lins[i].numel].view(lins[i].rows, lins[i].cols) for i in c],
                                       [S2[src]] * len(c), outs=[OUT[i] for i in c], dequant=False, run=False)
               for c in chunks]
        t_f6c = time_calls(lambda: [b.run() for b in FBc])
        del FBc
        t_mx = time_calls(lambda: [b.run() for b in MXB])
        t_mxn = time_calls(lambda: [b.run() for b in MXB_nodq])
        ACT6 = focus.quantize_act_per_token_fo6(X)
        t_a6 = time_calls(lambda: focus.quantize_act_per_token_fo6(X, out=ACT6), reps=20)
        t_mix = {t: time_calls(lambda t=t: [b.run() for b in MIXB[t]]) for t in MIX_TILES}
        del MAPS, MIXB, M32, MXB, MXB_nodq, FB
        # per-token activations on a tensor too large for any cache (1 GiB)
        XL = synth.make_activations((131072, 4096), device=dev)
        ACTL = focus.quantize_act_per_token(XL)
        t_al = time_calls(lambda: focus.quantize_act_per_token(XL, out=ACTL), reps=10)
        ACT6L = focus.quantize_act_per_token_fo6(XL)
        t_a6l = time_calls(lambda: focus.quantize_act_per_token_fo6(XL, out=ACT6L), reps=10)
        del XL, ACTL, ACT6L
        rows.update({
            "FourOverSix weights, codes only (after the steps)": row(t_f6, B_ACT * n_weights, n_weights),
            "FourOverSix weights, codes only, every linear reading the largest one's weights from the "
            "last-level cache (after the steps)": row(t_f6c, B_ACT * n_weights, n_weights),
            "FOCUS on MXFP4 + w' (after the steps)": row(t_mx, (B_MX + 2.0) * n_weights, n_weights),
            "FOCUS on MXFP4 codes only (after the steps)": row(t_mxn, B_MX * n_weights, n_weights),
            "FourOverSix act per token [8192,4096] (after the steps, cache-resident)":
                row(t_a6, B_ACT * X.numel() + 4 * X.shape[0], X.numel()),
            "act per token [131072,4096] (after the steps)":
                row(t_al, B_ACT * 131072 * 4096 + 4 * 131072, 131072 * 4096),
            "FourOverSix act per token [131072,4096] (after the steps)":
                row(t_a6l, B_ACT * 131072 * 4096 + 4 * 131072, 131072 * 4096),
        })
        for (th, tw) in MIX_TILES:
            share = synth.MIXFP4_FRAC[(th, tw)]
            rows[f"FlipQuant MixFP4 {th}x{tw} map ({100 * share:.2f}% E0M3 tiles) + w' (after the steps)"] = \
                row(t_mix[(th, tw)], (B_ACT + 2.0 + 1.0 / (th * tw)) * n_weights, n_weights)
    torch.cuda.synchronize()
    log("rows after the steps done")

    # ---- streaming ceiling: a hand-written kernel with the memory traffic of
    # one quantize + w' launch and none of its arithmetic, same process
    per_launch_blk = n_weights // 16 // nq
    t_sc, ceil_gbs, ceil_u = stream_ceiling(dev, per_launch_blk)
    rows[f"quantizer's traffic pattern without arithmetic, one launch's blocks, {ceil_u} per lane "
         f"(ceiling, after the steps)"] = row(t_sc, per_launch_blk * 85.0, per_launch_blk * 16)
    t_rc, _, rc_u, rc_g = read_ceiling(dev, per_launch_blk * 2)
    rows[f"tensor scale's traffic pattern without arithmetic, one launch's weights, {rc_u} loads per lane, "
         f"{rc_g} workgroups (ceiling, after the steps)"] = row(t_rc, per_launch_blk * 32.0, per_launch_blk * 16)
    t_dc, _ = deq_ceiling(dev, per_launch_blk)
    rows["dequantize's traffic pattern without arithmetic, one launch's blocks (ceiling, after the steps)"] = \
        row(t_dc, per_launch_blk * 41.0, per_launch_blk * 16)
    for tok in (8192, 131072):
        t_ac, _ = act_ceiling(dev, tok, 4096, reps=20 if tok == 8192 else 10)
        rows[f"per-token activation traffic without arithmetic [{tok},4096] (ceiling, after the steps)"] = \
            row(t_ac, B_ACT * tok * 4096 + 4 * tok, tok * 4096)
    # the activation phase's position in the step (right after the dequantize
    # phase, caches cold for X): the quantizer and the same traffic without
    # arithmetic, alternated over a few more steps
    t_pos = act_step_position(focus, R, X, ACT, dev)
    rows["act per token [8192,4096] in the step's position, alternated with the ceiling below (after the steps)"] = \
        row(t_pos[0], B_ACT * X.numel() + 4 * X.shape[0], X.numel())
    rows["per-token activation traffic without arithmetic [8192,4096] in the step's position (ceiling, after the steps)"] = \
        row(t_pos[1], B_ACT * X.numel() + 4 * X.shape[0], X.numel())
    csrc = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    t_cp = time_calls(lambda: cdst.copy_(csrc), reps=5)
    del csrc, cdst
    rows["runtime device copy 2 GiB (after the steps)"] = row(t_cp, 2.0 * (1 << 31), 1 << 31)

    if extra_rows:
        rows.update(linear_rows(focus, synth, ws, dev, stream))
        rows.update(decode_graph_row(focus, synth, ws, dev))
        rows.update(decode_layer_rows(focus, synth, ws, dev))
        rows.update(decode_layers_stream_row(focus, synth, ws, dev))
        log("linear-layer rows done")

    # ---- the Llama-3.2-1B-shaped set: the same step, with parity --------------
    par_1b = None
    if args.workload == "8b" and not args.no_1b:
        R1 = WeightSetRun(focus, synth, synth.LLAMA_1B, dev)
        for _ in range(args.warmup):
            R1.step()
        torch.cuda.synchronize()
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(4 * args.steps)]
        for k in range(args.steps):
            R1.step(lambda j, k=k: e1[4 * k + j].record(stream))
        torch.cuda.synchronize()
        ph1 = [sum(e1[4 * k + j].elapsed_time(e1[4 * k + j + 1]) for k in range(args.steps)) / args.steps
               for j in range(3)]
        step1 = sum(e1[4 * k].elapsed_time(e1[4 * k + 3]) for k in range(args.steps)) / args.steps
        n1 = R1.n_weights
        r1 = row(step1, (B_TENSOR_SCALE + B_QUANT_DQ + B_DEQUANT) * n1, n1)
        r1["quantize + w' ms"] = round(ph1[1], 4)
        r1["quantize + w' frac_hbm_peak"] = round(B_QUANT_DQ * n1 / (ph1[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        rows[f"{synth.LLAMA_1B.name} step: tensor_scale + quantize + w' + dequantize "
             f"(after the 8B rows)"] = r1
        log(f"1B set step {step1:.3f} ms")
        if not args.no_parity:
            par_1b, _ = check_set(R1, None, None, args, False, label="1B")
        del R1

    line = {
        "metric": METRIC if args.workload == "8b" else METRIC.replace("8B set", f"{args.workload.upper()} set"),
        "value": round(n_weights / (ms_step * 1e-3) / 1e9, 2),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"{ws.name}: {n_weights} BF16 weights; per step tensor_scale + quantize "
                        f"(codes, E4M3 scales, BF16 w') + dequantize for every linear, and per-token "
                        f"activations X [8192, 4096]"
                        + ("; w' and the dequantized copy to one reused per-layer buffer" if layered else ""),
            "weights": n_weights,
            "linears": nlin,
            "m": "LogNormal(0, 0.1)", "q": "N(6, 2)", "W": "N(0, %g) + 0.1%% outliers x20" % ws.std,
        },
        "quantize_gweights_s": round(n_weights / (phase["quantize_dq"] * 1e-3) / 1e9, 2),
        "quantize_codes_only_gweights_s": round(n_weights / (t_q * 1e-3) / 1e9, 2),
        "roofline": {
            "kernel": "focus_quantize (codes + scales + w')",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if args.workload == "8b" else None,
            "bytes_per_weight": B_QUANT_DQ,
            "weights_per_launch": round(n_weights / nq),
            "mean_launch_ms": round(mean_launch_ms, 5),
            "launches": len(q_launch_ms),
            "launches_per_step": nq,
            "timed_launches_in_trace": [args.warmup * nq, (args.warmup + args.steps) * nq],
            "stream_ceiling_GB_s": round(ceil_gbs, 1),
            "frac_of_ceiling": round(achieved / ceil_gbs, 4),
        },
        "parity": par,
        "parity_1b": par_1b,
        "cpu_baseline": cpu,
        "rows": rows,
        "wall_s_timed": round(wall, 3),
        "gpu_ms_timed": round(gpu_ms, 3),
    }
    print(json.dumps(line), flush=True)


def check_set(R, X, ACT, args, layered, label="8B"):
    """Every output of the last timed step against the oracle run on the same
    input bytes (copied to the host): s2 and amax of every linear, scale
    bytes, codes and w' (from the quantizer and from the dequantize call) of
    every linear, and the per-token activations.  Parity rule as in
    tests/parity.py: scales and s2 bit-exact, at most 1e-6 of the codes one
    step apart where sigmoid rounding explains it, w' exact where codes
    agree.  The layered 70B set checks layers 0, L/2 and L-1 (w' of the last
    layer only: the per-layer buffer is reused).  The oracle's quantize
    passes are timed (all host cores, row chunks) and give the CPU baseline.
    Returns (parity dict, cpu_baseline dict)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity as prule

    o = oracle.default()
    n_thr = prule.threads()
    lins = R.lins
    if layered:
        L = R.ws.layers
        keep = {0, L // 2, L - 1}
        todo = [i for i, l in enumerate(lins) if l.layer in keep]
        with_w = {i for i in todo if lins[i].layer == L - 1}
    else:
        todo = list(range(len(lins)))
        with_w = set(todo)
    limit = args.cpu_weights if args.cpu_weights > 0 else float("inf")
    S2h = R.S2.view(-1).cpu().numpy()
    AMh = R.AMAX.view(-1).cpu().numpy()

    def fetch(i):
        wb = synth.bits(R.W[i])
        h = {"wb": wb, "m": R.M[i].cpu().numpy(), "q": R.Q[i].cpu().numpy(),
             "codes": R.OUT[i].codes.cpu().numpy(), "scales": R.OUT[i].scales.cpu().numpy()}
        if i in with_w:
            h["wdq"] = synth.bits(R.WDQ[i])
            h["deq"] = synth.bits(R.DEQ[i])
        h["s2o"], h["amaxo"] = o.tensor_scale(wb)  # the oracle's own tensor scale
        return h

    tot = {"tensors": 0, "weights_checked": 0, "s2_mismatches": 0, "amax_mismatches": 0,
           "scale_mismatches": 0, "code_mismatches": 0, "wdeq_mismatches": 0, "dequantize_mismatches": 0,
           "wdeq_weights_checked": 0, "failures": []}
    oracle_s, oracle_w = 0.0, 0
    t_all = time.perf_counter()
    with ThreadPoolExecutor(n_thr) as pool, ThreadPoolExecutor(1) as pre:
        nxt = pre.submit(fetch, todo[0]) if todo else None
        for pos, i in enumerate(todo):
            if tot["weights_checked"] >= limit:
                break
            h = nxt.result()
            nxt = pre.submit(fetch, todo[pos + 1]) if pos + 1 < len(todo) else None
            rows = lins[i].rows
            dq = "wdq" in h
            bounds = np.linspace(0, rows, min(n_thr, rows) + 1).astype(int)
            parts = [(bounds[k], bounds[k + 1]) for k in range(len(bounds) - 1) if bounds[k + 1] > bounds[k]]
            t0 = time.perf_counter()
            refs = list(pool.map(lambda ab: o.quantize(h["wb"][ab[0]:ab[1]], h["m"][ab[0]:ab[1]],
                                                       h["q"][ab[0]:ab[1]], h["s2o"], dq), parts))
            oracle_s += time.perf_counter() - t0
            oracle_w += lins[i].numel

            def compare(k):
                a, b = parts[k]
                codes, scales, wdq = refs[k]
                out = {"scale": int(np.count_nonzero(h["scales"][a:b] != scales)), "code": 0, "wdq": 0,
                       "deq": 0, "err": None}
                if np.array_equal(h["codes"][a:b], codes):
                    agree = None
                else:
                    try:  # the full rule: one step, explained by sigmoid rounding, within 1e-6
                        st = prule.check_quantized(o, h["wb"][a:b], h["m"][a:b], h["q"][a:b], h["s2o"],
                                                   h["codes"][a:b], h["scales"][a:b],
                                                   h["wdq"][a:b] if dq else None, ref=refs[k],
                                                   label=f"{label} linear {i} rows {a}:{b}",
                                                   count_limit=(b - a) * h["codes"].shape[1] * 2)
                        out["code"] = st["code_mismatches"]
                    except AssertionError as e:
                        out["err"] = str(e)[:300]
                        out["code"] = -1
                    agree = (prule.unpack(h["codes"][a:b]) == prule.unpack(codes))
                if dq:
                    for key, name in (("wdq", "wdq"), ("deq", "deq")):
                        diff = h[key][a:b] != wdq
                        if agree is not None:
                            diff &= agree
                        out[name] = int(np.count_nonzero(diff))
                return out

            res = list(pool.map(compare, range(len(parts))))
            tot["tensors"] += 1
            tot["weights_checked"] += lins[i].numel
            if dq:
                tot["wdeq_weights_checked"] += lins[i].numel
            if S2h[i].view(np.uint32) != np.float32(h["s2o"]).view(np.uint32):
                tot["s2_mismatches"] += 1
            if AMh[i].view(np.uint32) != np.float32(h["amaxo"]).view(np.uint32):
                tot["amax_mismatches"] += 1
            for r in res:
                tot["scale_mismatches"] += r["scale"]
                tot["code_mismatches"] += max(r["code"], 0)
                tot["wdeq_mismatches"] += r["wdq"]
                tot["dequantize_mismatches"] += r["deq"]
                if r["err"] and len(tot["failures"]) < 4:
                    tot["failures"].append(r["err"])
            if pos % 16 == 15 or pos == len(todo) - 1:
                log(f"{label} parity: {tot['tensors']}/{len(todo)} linears, {tot['weights_checked']} weights, "
                    f"{time.perf_counter() - t_all:.0f} s")
        if X is not None:
            xb = synth.bits(X)
            codes, scales, s2t, _ = prule.oracle_act_rows(o, xb, dequant=False, n_threads=n_thr)
            tot["act_tokens"] = int(xb.shape[0])
            tot["act_scale_mismatches"] = int(np.count_nonzero(ACT.scales.cpu().numpy() != scales))
            tot["act_code_mismatches"] = int(np.count_nonzero(prule.unpack(ACT.codes.cpu().numpy()) !=
                                                              prule.unpack(codes)))
            tot["act_s2_mismatches"] = int(np.count_nonzero(ACT.s2.cpu().numpy().view(np.uint32) !=
                                                            s2t.view(np.uint32)))
    allowed = int(np.floor(prule.CODE_MISMATCH_RATE * tot["weights_checked"]))
    tot["code_mismatches_allowed"] = allowed
    tot["seconds"] = round(time.perf_counter() - t_all, 1)
    tot["ok"] = (not tot["failures"] and tot["s2_mismatches"] == 0 and tot["amax_mismatches"] == 0 and
                 tot["scale_mismatches"] == 0 and tot["code_mismatches"] <= allowed and
                 tot["wdeq_mismatches"] == 0 and tot["dequantize_mismatches"] == 0 and
                 tot.get("act_scale_mismatches", 0) == 0 and tot.get("act_code_mismatches", 0) == 0 and
                 tot.get("act_s2_mismatches", 0) == 0)
    if not tot["failures"]:
        del tot["failures"]
    log(f"{label} parity: {'ok' if tot['ok'] else 'FAILED'} in {tot['seconds']} s")
    cpu = None
    if oracle_w:
        # one core: the oracle's quantize on the first 32 M weights of the set
        wb = synth.bits(R.W[0])
        r1 = max(1, min(wb.shape[0], (1 << 25) // wb.shape[1]))
        s2o, _ = o.tensor_scale(wb)
        m1, q1 = R.M[0][:r1].cpu().numpy(), R.Q[0][:r1].cpu().numpy()
        t1 = time.perf_counter()
        o.quantize(wb[:r1], m1, q1, s2o, True)
        per_core = r1 * wb.shape[1] / (time.perf_counter() - t1) / 1e9
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
        except OSError:
            pass
        cpu = {"value": round(oracle_w / oracle_s / 1e9, 5), "unit": "Gweights/s", "cores": n_thr,
               "per_core_value": round(per_core, 5), "cpu_model": model, "kind": "oracle",
               "seconds": round(oracle_s, 2),
               "sample": f"the oracle's quantize (codes, E4M3 scales, w') of {oracle_w} weights "
                         f"({tot['tensors']} linears of the {R.ws.name}, whole tensors, row chunks on "
                         f"{n_thr} host threads), on the same input bytes as the GPU; the same pass "
                         f"is the parity check"}
    return tot, cpu


def linear_rows(focus, synth, ws, dev, stream):
    """The NVFP4 linear layer Y = X' W'^T on each distinct layer shape of the
    set: 8192 tokens and 2048 tokens (one evaluation window; matrix-core
    bound, FLOP/s against the FP16 peak) and 16 tokens (bound by streaming W;
    operand bytes against the HBM peak).  Each shape is timed over repeated
    calls of the C ABI with prepared arguments and the split-k workspace the
    library asks for; the operands are random NVFP4 bytes."""
    import torch
    lib = focus._lib.lib()
    out = {}
    shapes = sorted(set(ws.layer_shapes()))
    for m_tok, reps in ((8192, 10), (2048, 20), (16, 50)):
        tot_ms, tot_flop, tot_bytes = 0.0, 0.0, 0.0
        for n, k in shapes:
            xc, xs = synth.nvfp4_operand(m_tok, k, seed=3, tensor_id=60, device=dev)
            wc, wsc = synth.nvfp4_operand(n, k, seed=3, tensor_id=61, device=dev)
            s2x = torch.full((m_tok,), 1e-3, dtype=torch.float32, device=dev)
            s2w = torch.full((1,), 1e-3, dtype=torch.float32, device=dev)
            y = torch.empty((m_tok, n), dtype=torch.bfloat16, device=dev)
            nws = int(lib.focus_nvfp4_linear_workspace_bytes(m_tok, n, k))
            wsp = torch.empty(max(nws // 4, 1), dtype=torch.float32, device=dev)
            args = (xc.data_ptr(), xs.data_ptr(), s2x.data_ptr(), 1, m_tok, wc.data_ptr(), wsc.data_ptr(),
                    s2w.data_ptr(), n, k, y.data_ptr(), 1, wsp.data_ptr(), nws, stream.cuda_stream)
            for _ in range(3):
                focus._lib.check(lib.focus_nvfp4_linear(*args))
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                lib.focus_nvfp4_linear(*args)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            tot_ms += ms
            tot_flop += 2.0 * m_tok * n * k
            tot_bytes += (m_tok + n) * k * 0.5625 + 2.0 * m_tok * n
            del xc, xs, wc, wsc, y, wsp
        tflops = tot_flop / (tot_ms * 1e-3) / 1e12
        gbs = tot_bytes / (tot_ms * 1e-3) / 1e9
        key = f"NVFP4 linear Y = X' W'^T, {m_tok} tokens through the {len(shapes)} layer shapes (after the steps)"
        out[key] = {"ms": round(tot_ms, 4), "TFLOP_s": round(tflops, 1),
                    "frac_mfma_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                    "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def decode_graph_row(focus, synth, ws, dev, m_tok=16, reps=50):
    """The 16-token linear layer on the distinct layer shapes, the four calls
    captured once in sequence in a HIP graph and replayed: unlike the row
    above, which times each shape over repeated identical calls (whose
    launches overlap a little), every kernel here follows a different one,
    as in a decode pass through the layers."""
    import torch
    lib = focus._lib.lib()
    shapes = sorted(set(ws.layer_shapes()))
    keep = []
    for n, k in shapes:
        xc, xs = synth.nvfp4_operand(m_tok, k, seed=3, tensor_id=60, device=dev)
        wc, wsc = synth.nvfp4_operand(n, k, seed=3, tensor_id=61, device=dev)
        s2x = torch.full((m_tok,), 1e-3, dtype=torch.float32, device=dev)
        s2w = torch.full((1,), 1e-3, dtype=torch.float32, device=dev)
        y = torch.empty((m_tok, n), dtype=torch.bfloat16, device=dev)
        nws = int(lib.focus_nvfp4_linear_workspace_bytes(m_tok, n, k))
        wsp = torch.empty(max(nws // 4, 1), dtype=torch.float32, device=dev)
        keep.append((xc, xs, s2x, wc, wsc, s2w, y, wsp, n, k, nws))

    def calls(stream_handle):
        for xc, xs, s2x, wc, wsc, s2w, y, wsp, n, k, nws in keep:
            focus._lib.check(lib.focus_nvfp4_linear(xc.data_ptr(), xs.data_ptr(), s2x.data_ptr(), 1, m_tok,
                                                    wc.data_ptr(), wsc.data_ptr(), s2w.data_ptr(), n, k,
                                                    y.data_ptr(), 1, wsp.data_ptr(), nws, stream_handle))

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls(side.cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flop = sum(2.0 * m_tok * n * k for n, k in shapes)
    byts = sum((m_tok + n) * k * 0.5625 + 2.0 * m_tok * n for n, k in shapes)
    key = (f"NVFP4 linear Y = X' W'^T, {m_tok} tokens, the {len(shapes)} layer shapes in sequence, "
           "one HIP graph replay (after the steps)")
    del graph, keep
    return {key: {"ms": round(ms, 4), "TFLOP_s": round(flop / (ms * 1e-3) / 1e12, 1),
                  "GB_s": round(byts / (ms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def decode_layer_rows(focus, synth, ws, dev, m_tok=16, reps=50):
    """One decoder layer's seven linears at 16 tokens, captured once in a HIP
    graph and replayed: q, k and v share the attention input, gate and up the
    MLP input, so the layer is grouped(q, k, v), o, grouped(gate, up), down
    (four launches); the same seven linears as seven single calls for
    comparison.  Operand bytes: codes and scales of X and W (0.5625 B per
    element) and the BF16 outputs."""
    import torch
    h, kv, f = ws.hidden, ws.kv, ws.inter

    def w(n, k, tid):
        c, s = synth.nvfp4_operand(n, k, seed=5, tensor_id=tid, device=dev)
        return focus.Quantized(c, s, None, torch.full((1,), 1e-3, dtype=torch.float32, device=dev))

    def x(k, tid):
        c, s = synth.nvfp4_operand(m_tok, k, seed=5, tensor_id=tid, device=dev)
        return focus.Quantized(c, s, None, torch.full((m_tok,), 1e-3, dtype=torch.float32, device=dev))

    xa, xo, xm, xd = x(h, 70), x(h, 71), x(h, 72), x(f, 73)
    q, k, v, o = w(h, h, 80), w(kv, h, 81), w(kv, h, 82), w(h, h, 83)
    gate, up, down = w(f, h, 84), w(f, h, 85), w(h, f, 86)
    calls = [(xa, [q, k, v]), (xo, [o]), (xm, [gate, up]), (xd, [down])]
    outs = [[torch.empty((m_tok, wt.codes.shape[0]), dtype=torch.bfloat16, device=dev) for wt in g] for _, g in calls]
    wsp = {}
    for xx, g in calls:
        for wt in g:
            n_ = int(focus.nvfp4_linear_workspace_bytes(m_tok, wt.codes.shape[0], xx.codes.shape[1] * 2))
            wsp[id(wt)] = torch.empty(max(n_ // 4, 1), dtype=torch.float32, device=dev) if n_ else None

    def grouped():
        for (xx, g), og in zip(calls, outs):
            if len(g) == 1:
                focus.nvfp4_linear(xx, g[0], out=og[0], workspace=wsp[id(g[0])])
            else:
                focus.nvfp4_linear_grouped(xx, g, outs=og, workspace=None)

    def single():
        for (xx, g), og in zip(calls, outs):
            for wt, yy in zip(g, og):
                focus.nvfp4_linear(xx, wt, out=yy, workspace=wsp[id(wt)])

    nbytes = sum((m_tok + sum(wt.codes.shape[0] for wt in g)) * xx.codes.shape[1] * 2 * 0.5625 +
                 2.0 * m_tok * sum(wt.codes.shape[0] for wt in g) for xx, g in calls)
    flop = sum(2.0 * m_tok * wt.codes.shape[0] * xx.codes.shape[1] * 2 for xx, g in calls for wt in g)
    res = {}
    for name, fn, launches in (("grouped (4 launches)", grouped, 4), ("seven single calls", single, 7)):
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        key = (f"NVFP4 linear, one {ws.name.split(' (')[0]} layer (q, k, v, o, gate, up, down) at {m_tok} tokens, "
               f"{name}, one HIP graph replay (after the steps)")
        res[key] = {"ms": round(ms, 4), "TFLOP_s": round(flop / (ms * 1e-3) / 1e12, 1), "GB_s": round(gbs, 1),
                    "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del graph
    return res



def decode_layers_stream_row(focus, synth, ws, dev, m_tok=16, n_layers=8, reps=20):
    """Eight distinct decoder layers at 16 tokens, each as the four grouped
    launches of decode_layer_rows, captured in one HIP graph and replayed;
    reported per layer.  The rows above re-read one shape's (or one layer's)
    weights on every call, which then stay in the 256 MB Infinity Cache (the
    small ones in L2); eight layers hold about 1 GB of weights, so each layer
    streams its weights from HBM, as in a decode pass through the model."""
    import torch
    h, kv, f = ws.hidden, ws.kv, ws.inter

    def op(rows, k, tid, per_row):
        c, s = synth.nvfp4_operand(rows, k, seed=6, tensor_id=tid, device=dev)
        return focus.Quantized(c, s, None, torch.full((rows if per_row else 1,), 1e-3, dtype=torch.float32,
                                                      device=dev))

    layers = []
    for li in range(n_layers):
        t0 = 100 + 16 * li
        xa, xo, xm, xd = (op(m_tok, h, t0, True), op(m_tok, h, t0 + 1, True), op(m_tok, h, t0 + 2, True),
                          op(m_tok, f, t0 + 3, True))
        q, k, v, o = op(h, h, t0 + 4, False), op(kv, h, t0 + 5, False), op(kv, h, t0 + 6, False), op(h, h, t0 + 7, False)
        gate, up, down = op(f, h, t0 + 8, False), op(f, h, t0 + 9, False), op(h, f, t0 + 10, False)
        calls = [(xa, [q, k, v]), (xo, [o]), (xm, [gate, up]), (xd, [down])]
        outs = [[torch.empty((m_tok, wt.codes.shape[0]), dtype=torch.bfloat16, device=dev) for wt in g]
                for _, g in calls]
        wsp = {}
        for xx, g in calls:
            if len(g) == 1:
                n_ = int(focus.nvfp4_linear_workspace_bytes(m_tok, g[0].codes.shape[0], xx.codes.shape[1] * 2))
                wsp[id(g[0])] = torch.empty(max(n_ // 4, 1), dtype=torch.float32, device=dev) if n_ else None
        layers.append((calls, outs, wsp))
    nbytes = sum((m_tok + sum(wt.codes.shape[0] for wt in g)) * xx.codes.shape[1] * 2 * 0.5625 +
                 2.0 * m_tok * sum(wt.codes.shape[0] for wt in g) for xx, g in layers[0][0])
    wbytes = n_layers * sum(wt.codes.numel() + wt.scales.numel() for _, g in layers[0][0] for wt in g)

    def run():
        for calls, outs, wsp in layers:
            for (xx, g), og in zip(calls, outs):
                if len(g) == 1:
                    focus.nvfp4_linear(xx, g[0], out=og[0], workspace=wsp[id(g[0])])
                else:
                    focus.nvfp4_linear_grouped(xx, g, outs=og, workspace=None)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps / n_layers
    gbs = nbytes / (ms * 1e-3) / 1e9
    key = (f"NVFP4 linear, {n_layers} distinct {ws.name.split(' (')[0]} layers at {m_tok} tokens "
           f"({wbytes / 1e9:.2f} GB of weights, beyond the Infinity Cache), grouped, one HIP graph replay, "
           "per layer (after the steps)")
    del graph, layers
    return {key: {"ms": round(ms, 4), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}}


if __name__ == "__main__":
    main()
