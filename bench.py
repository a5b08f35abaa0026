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
second of step time).  ``roofline`` reports the dominant kernel,
focus_quantize with w', against the 8 TB/s HBM peak: algorithmic bytes
(5.3125 B per weight) / mean launch duration, every launch bracketed by HIP
events on the stream it runs on.  ``rows`` breaks the step down per call and
adds the codes-only quantize (3.3125 B per weight) timed after the steps.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b|1b]
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-weights", type=float, default=1.6e9,
                    help="weights of the set (in linear order) the CPU oracle quantizes")
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
    lins = ws.linears()
    n_weights = sum(l.numel for l in lins)

    # ---- inputs (resident in HBM) and outputs ----------------------------
    t0 = time.time()
    W, M, Q = [], [], []
    for lin in lins:
        w, m, q = synth.make_linear(ws, lin, device=dev)
        W.append(w)
        M.append(m)
        Q.append(q)
    X = synth.make_activations(device=dev)
    S2 = torch.empty((len(lins), 1), dtype=torch.float32, device=dev)
    AMAX = torch.empty((len(lins), 1), dtype=torch.float32, device=dev)
    if layered:
        # w' and the dequantized copy of one layer at a time: every layer's
        # linears are views of one reused buffer each
        per_layer = max(sum(l.numel for l in lins if l.layer == k) for k in range(ws.layers))
        wdq_buf = torch.empty(per_layer, dtype=torch.bfloat16, device=dev)
        deq_buf = torch.empty(per_layer, dtype=torch.bfloat16, device=dev)
        WDQ, DEQ, off = [], [], {}
        for l in lins:
            o = off.get(l.layer, 0)
            WDQ.append(wdq_buf[o:o + l.numel].view(l.rows, l.cols))
            DEQ.append(deq_buf[o:o + l.numel].view(l.rows, l.cols))
            off[l.layer] = o + l.numel
    else:
        WDQ = [torch.empty((l.rows, l.cols), dtype=torch.bfloat16, device=dev) for l in lins]
        DEQ = [torch.empty((l.rows, l.cols), dtype=torch.bfloat16, device=dev) for l in lins]
    OUT = [focus.Quantized(torch.empty((l.rows, l.cols // 2), dtype=torch.uint8, device=dev),
                           torch.empty((l.rows, l.cols // 16), dtype=torch.uint8, device=dev),
                           WDQ[i], S2[i]) for i, l in enumerate(lins)]
    ACT = focus.quantize_act_per_token(X)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"# generated {ws.name}: {n_weights} weights in {gen_s:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    nlin = len(lins)

    # Prepared batched calls, 32 linears each: every quantize / dequantize
    # batch is exactly one kernel launch, every tensor-scale batch three.
    if layered:
        chunks = [[i for i, l in enumerate(lins) if l.layer == k] for k in range(ws.layers)]
    else:
        chunks = [list(range(i, min(i + 32, nlin))) for i in range(0, nlin, 32)]
    TS = [focus.tensor_scale_many([W[i] for i in c], S2[c[0]:c[-1] + 1], AMAX[c[0]:c[-1] + 1], run=False)
          for c in chunks]
    QB = [focus.quantize_many([W[i] for i in c], [M[i] for i in c], [Q[i] for i in c], [S2[i] for i in c],
                              outs=[OUT[i] for i in c], dequant=True, run=False) for c in chunks]
    QB_nodq = [focus.quantize_many([W[i] for i in c], [M[i] for i in c], [Q[i] for i in c],
                                   [S2[i] for i in c], outs=[OUT[i] for i in c], dequant=False, run=False)
               for c in chunks]
    extra_rows = not layered
    FB = [] if not extra_rows else [focus.quantize_fo6_many([W[i] for i in c], [S2[i] for i in c], outs=[OUT[i] for i in c],
                                  dequant=False, run=False) for c in chunks]
    M32 = [] if not extra_rows else [
        synth.block_factor_lognormal((l.rows, l.cols // 32), seed=42, tensor_id=l.tid(1), device=dev)
        for l in lins]
    MXB = [] if not extra_rows else [focus.quantize_mx_many([W[i] for i in c], [M32[i] for i in c], [Q[i] for i in c],
                                  outs=[focus.Quantized(OUT[i].codes, OUT[i].scales.view(-1)[:lins[i].numel // 32]
                                                        .view(lins[i].rows, lins[i].cols // 32), OUT[i].deq, None)
                                        for i in c], dequant=True, run=False) for c in chunks]
    MXB_nodq = [] if not extra_rows else [focus.quantize_mx_many([W[i] for i in c], [M32[i] for i in c], [Q[i] for i in c],
                                       outs=[focus.Quantized(OUT[i].codes,
                                                             OUT[i].scales.view(-1)[:lins[i].numel // 32]
                                                             .view(lins[i].rows, lins[i].cols // 32), None, None)
                                             for i in c], dequant=False, run=False) for c in chunks]
    MIX_TILES = [(8, 64), (16, 64), (256, 64)]
    MAPS = {} if not extra_rows else {
        t: [synth.tile_map(l.rows, l.cols, t, frac=synth.MIXFP4_FRAC[t], seed=42, tensor_id=l.tid(3), device=dev)
            for l in lins] for t in MIX_TILES}
    MIXB = {} if not extra_rows else {
        t: [focus.quantize_mixfp4_many([W[i] for i in c], [MAPS[t][i] for i in c], [t] * len(c),
                                       [S2[i] for i in c], outs=[OUT[i] for i in c], dequant=True, run=False)
            for c in chunks] for t in MIX_TILES}
    DB = [focus.dequantize_many([OUT[i].codes for i in c], [OUT[i].scales for i in c], [S2[i] for i in c],
                                outs=[DEQ[i] for i in c], run=False) for c in chunks]
    nq = len(QB)

    # events of one step: [0] start, [1] tensor scales done, a pair around
    # each quantize launch, quantize phase done, dequantize done, act done
    n_ev = 5 + 2 * nq
    E_TS, E_Q0, E_QEND, E_DQ, E_ACT = 1, 2, 2 + 2 * nq, 3 + 2 * nq, 4 + 2 * nq

    def step(ev=None):
        rec = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        rec(0)
        for b in TS:
            b.run()
        rec(E_TS)
        for i, b in enumerate(QB):
            rec(E_Q0 + 2 * i)
            b.run()
            rec(E_Q0 + 2 * i + 1)
        rec(E_QEND)
        for b in DB:
            b.run()
        rec(E_DQ)
        focus.quantize_act_per_token(X, out=ACT)
        rec(E_ACT)

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

    t_q = time_calls(lambda: [b.run() for b in QB_nodq])
    if extra_rows:
        t_f6 = time_calls(lambda: [b.run() for b in FB])
        t_mx = time_calls(lambda: [b.run() for b in MXB])
        t_mxn = time_calls(lambda: [b.run() for b in MXB_nodq])
        ACT6 = focus.quantize_act_per_token_fo6(X)
        t_a6 = time_calls(lambda: focus.quantize_act_per_token_fo6(X, out=ACT6), reps=20)
        t_mix = {t: time_calls(lambda t=t: [b.run() for b in MIXB[t]]) for t in MIX_TILES}
        # per-token activations on a tensor too large for any cache (1 GiB)
        XL = synth.make_activations((131072, 4096), device=dev)
        ACTL = focus.quantize_act_per_token(XL)
        t_al = time_calls(lambda: focus.quantize_act_per_token(XL, out=ACTL), reps=10)
        del XL, ACTL
    torch.cuda.synchronize()

    def row(ms, nbytes, units):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "Gunits_s": round(units / (ms * 1e-3) / 1e9, 2)}

    rows = {
        "tensor_scale (step phase)": row(phase["tensor_scale"], B_TENSOR_SCALE * n_weights, n_weights),
        "quantize + w' (step phase)": row(phase["quantize_dq"], B_QUANT_DQ * n_weights, n_weights),
        "dequantize (step phase)": row(phase["dequantize"], B_DEQUANT * n_weights, n_weights),
        "act per token [8192,4096] (step phase)": row(phase["act"], B_ACT * X.numel() + 4 * X.shape[0],
                                                      X.numel()),
        "quantize codes only (after the steps)": row(t_q, B_QUANT * n_weights, n_weights),
    }
    if extra_rows:
        rows.update({
            "FourOverSix weights, codes only (after the steps)": row(t_f6, B_ACT * n_weights, n_weights),
            "FOCUS on MXFP4 + w' (after the steps)": row(t_mx, (B_MX + 2.0) * n_weights, n_weights),
            "FOCUS on MXFP4 codes only (after the steps)": row(t_mxn, B_MX * n_weights, n_weights),
            "FourOverSix act per token [8192,4096] (after the steps, cache-resident)":
                row(t_a6, B_ACT * X.numel() + 4 * X.shape[0], X.numel()),
        })
        rows["act per token [131072,4096] (after the steps)"] = row(t_al, B_ACT * 131072 * 4096 + 4 * 131072,
                                                                     131072 * 4096)
        for (th, tw) in MIX_TILES:
            share = synth.MIXFP4_FRAC[(th, tw)]
            rows[f"FlipQuant MixFP4 {th}x{tw} map ({100 * share:.2f}% E0M3 tiles) + w' (after the steps)"] = \
                row(t_mix[(th, tw)], (B_ACT + 2.0 + 1.0 / (th * tw)) * n_weights, n_weights)

    # streaming ceiling on this GPU: a plain device copy of 2 GiB (read + write)
    csrc = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    t_cp = time_calls(lambda: cdst.copy_(csrc), reps=5)
    del csrc, cdst
    copy_gbs = 2.0 * (1 << 31) / (t_cp * 1e-3) / 1e9
    rows["device copy 2 GiB (streaming ceiling, after the steps)"] = row(t_cp, 2.0 * (1 << 31), 1 << 31)
    if extra_rows:
        rows.update(linear_rows(focus, synth, ws, dev, stream))
        rows.update(decode_graph_row(focus, synth, ws, dev))

    # ---- CPU baseline: the oracle on a bounded sample ----------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lins, W, M, Q, X, args.cpu_weights)

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
        "roofline": {
            "kernel": "focus_quantize (codes + scales + w')",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if args.workload == "8b" else None,
            "bytes_per_weight": B_QUANT_DQ,
            "mean_launch_ms": round(mean_launch_ms, 5),
            "launches": len(q_launch_ms),
            "launches_per_step": nq,
            "copy_ceiling_GB_s": round(copy_gbs, 1),
            "frac_of_copy_ceiling": round(achieved / copy_gbs, 4),
        },
        "cpu_baseline": cpu,
        "rows": rows,
        "wall_s_timed": round(wall, 3),
        "gpu_ms_timed": round(gpu_ms, 3),
    }
    print(json.dumps(line), flush=True)


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


def cpu_baseline(lins, W, M, Q, X, budget):
    """The oracle, unchanged, on the first `budget` weights of the set in
    linear order (whole tensors, the last one cut by rows): s2 of each full
    tensor, then quantize (+ w') and dequantize, and per-token activations of
    the first 512 tokens; row chunks run on the host's cores through ctypes
    (which releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    o = oracle.default()
    try:
        n_thr = len(os.sched_getaffinity(0))
    except AttributeError:
        n_thr = os.cpu_count() or 1
    n_thr = max(1, min(n_thr, 64))
    host, left = [], int(budget)
    for i, lin in enumerate(lins):
        if left <= 0:
            break
        wb = synth.bits(W[i])
        r = max(1, min(lin.rows, left // lin.cols))
        host.append((wb, M[i][:r].cpu().numpy(), Q[i][:r].cpu().numpy(), r))
        left -= r * lin.cols
    xb = synth.bits(X[:512])
    weights = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(n_thr) as ex:
        for wb, m, q, r in host:
            s2, _ = o.tensor_scale(wb)
            bounds = np.linspace(0, r, n_thr + 1).astype(int)

            def work(k, wb=wb, m=m, q=q, s2=s2, bounds=bounds):
                a, b = bounds[k], bounds[k + 1]
                if b <= a:
                    return 0
                codes, scales, _ = o.quantize(wb[a:b], m[a:b], q[a:b], s2, True)
                o.dequantize(codes, scales, s2)
                return (b - a) * wb.shape[1]

            weights += sum(ex.map(work, range(n_thr)))
        tb = np.linspace(0, xb.shape[0], n_thr + 1).astype(int)
        list(ex.map(lambda k: o.quantize_act_per_token(xb[tb[k]:tb[k + 1]]), range(n_thr)))
    dt = time.perf_counter() - t0
    # one core: the first 32 M weights of the same sample on one thread
    wb, m, q, r = host[0]
    r1 = max(1, min(r, (1 << 25) // wb.shape[1]))
    s2, _ = o.tensor_scale(wb)
    t1 = time.perf_counter()
    codes, scales, _ = o.quantize(wb[:r1], m[:r1], q[:r1], s2, True)
    o.dequantize(codes, scales, s2)
    per_core = r1 * wb.shape[1] / (time.perf_counter() - t1) / 1e9
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": round(weights / dt / 1e9, 5), "unit": "Gweights/s", "cores": n_thr,
            "per_core_value": round(per_core, 5), "cpu_model": model,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"the first {weights} weights of the set in linear order ({len(host)} linears, the "
                      f"last cut by rows): full-tensor s2, then quantize (+w') and dequantize, and "
                      f"per-token activations of 512 x 4096"}


if __name__ == "__main__":
    main()
