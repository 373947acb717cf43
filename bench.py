#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step = one pass of every row of the hot path over the training-step
linear workload at the Llama-7B MLP shapes, for both orientations of the
weight (gate/up W 11008x4096 and down W 4096x11008; bf16 Student-t(5)
weights scaled to std 0.02, M = 2048 tokens, LoRA r = 16, alpha = 32):

  quantise  nf4_quantize_dq_batch of both bf16 weights (quantise +
            double-quantise of the two in one launch)
  dequant   nf4_dequant to bf16 (the standalone bit-exact expansion)
  gemm      qlora_linear_fwd    at M = 2048 with r = 0: exactly one launch
            of the fused dequant GEMM kernel per call (the roofline kernel)
  fwd       qlora_linear_fwd    at M = 2048 (LoRA-down + fused dequant GEMM)
  bwd       qlora_linear_bwd_dx at M = 2048 (B^T, LoRA t + fused dequant GEMM)
  grads     lora_grads with the saved u, t
  merge     qlora_merge: the merged bf16 weight dequant(W) + (alpha/r) B A
  gemv      qlora_linear_fwd at M = 1, 4, 16 (decode: LoRA-down + dequant
            GEMV), over rotating quantised copies totalling >= 512 MiB so no
            call is served from the 256 MiB Infinity Cache.  The decode calls
            are captured once in HIP graphs (one per shape and M) and the
            graphs are replayed each step: at 6-15 us per call, eager Python
            launches would measure the host, not the GPU.

The decode graphs also cover the q_proj decode shape, W 4096x4096
N(0, 0.02) (its own rotating copies, x, A, B from the same recipe), and
each shape at M = 1 without the LoRA term (r = 0: the GEMV kernel is then
the whole call; "gemv.kernel_only_r0").

"decode_layer_7b" times one token (M = 1, r = 16) through the seven
projections of a 7B-shaped layer, captured in one HIP graph over rotating
layer copies beyond the Infinity Cache: microseconds per layer, and the
32-layer product (linear layers only); "stacked" is the same layer as four
calls, q|k|v and gate|up each one call on row-stacked weights and adapters.

After the K steps, "layer_7b" times a full 7B-shaped decoder layer (q, k,
v, o 4096x4096; gate, up 11008x4096; down 4096x11008), its weights bf16
N(0, 0.02) drawn and quantised on the device: quantise + DQ (one launch), fwd, bwd_dx
and lora_grads of all seven at M = 2048, r = 64, alpha = 16.  "layer_65b"
times fwd and bwd_dx of the 65B-shaped layer (8192 hidden, 22016 MLP, bf16
N(0, 0.015)) at M = 4096, r = 64, alpha = 16.  "hbm_measured" gives the
streaming-read rate of qn_hbm_read_probe (16-byte loads, read only) and
the copy and read rates of plain torch kernels on 1 GiB, as context for the
fractions of the 8 TB/s peak.

"quantise_65b" times the quantiser (nf4_quantize_dq_batch, one launch per
layer) over 80 layers of the 65B shapes (7 projections, 809.5M weights per
layer): 8 distinct device-resident layers of bf16 N(0, 0.015) weights
(torch's generator, seed 5; each layer is 1.6 GB, far beyond the Infinity
Cache) quantised in turn 10 times over.

"adamw_7b_lora" times lora_adamw_step over all 40 M LoRA parameters of a
7B model at r = 16 (seven projections x 32 layers).

"dropout" times LoRA dropout (p = 0.05) on the same two training-step
linears: lora_dropout of x (2048 x 4096 or 2048 x 11008 bf16, read once and
written once) and the forward / backward-to-input calls with dropout,
against the same calls without it.

"unfused_context" times, as context only, the unfused way of doing the
same base products: nf4_dequant to bf16 in HBM, then torch's bf16 GEMM.

Inputs are resident in HBM before the timed region.  Every phase is timed
with HIP events on the stream the library launches on (torch's current
stream); the K timed steps are bracketed by synchronisations.

JSON line: value = dequant-GEMM TFLOP/s (2 M N K + LoRA flops of the fwd and
bwd calls over their event time).  "gemv" holds the decode GB/s at
4096x11008 (the metric's shape) and the other shapes / M.  "roofline" is the
dominant kernel: the fused dequant GEMM, timed per launch from the "gemm"
phase (a call with r = 0 is one GEMM launch and nothing else; with r = 16 a
call adds the LoRA-down kernels and a 16-deep LoRA step, 0.5% of the flops);
"traffic" comes from the committed PMC summary when its kernel source hash
still matches.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dequant-GEMM TFLOP/s + dequant-GEMV GB/s (% roofline) at 4096x11008 NF4"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
SHAPES = [(11008, 4096), (4096, 11008)]
M_TRAIN, RANK, ALPHA = 2048, 16, 32.0
DECODE_M = (1, 4, 16)
DECODE_SQUARE = (4096, 4096)   # the q_proj decode shape, W ~ N(0, 0.02)
LAYER7B = dict(M=2048, r=64, alpha=16.0, std=0.02, seed=6)
LAYER65B = dict(M=4096, r=64, alpha=16.0, std=0.015, seed=8)
GEMV_HEADLINE = (4096, 11008, 1)
ROTATE_BYTES = 512 << 20
Q65_LAYERS, Q65_DISTINCT = 80, 8
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_fwd_mlp_shapes_m2048_pmc.md")
GEMM_SOURCE = os.path.join(ROOT, "bit_nf4_quantized_22_amd", "csrc", "qn_gemm.hip")

BYTES_PER_WEIGHT = 0.5 + 1 / 64 + 4 / (64 * 256)  # NF4 codes + q8 + c2


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run plain 256 MiB device copies (PMC counter calibration)")
    return p.parse_args()


def gemv_bytes(N, K, M, r):
    """Algorithmic HBM bytes of one decode call: the quantised weight, A and
    B, x in and y out."""
    return N * K * BYTES_PER_WEIGHT + 2 * r * (N + K) + 2 * M * (K + N)


def linear_flops(N, K, M, r):
    return 2.0 * M * N * K + 2.0 * M * r * (N + K)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic():
    """HBM bytes per GEMM launch from the committed PMC summary, or None if
    it is missing or was taken on a different GEMM source."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    h = re.search(r"gemm source sha256/16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != source_hash(GEMM_SOURCE):
        return None
    return float(b.group(1))


def cpu_baseline(workloads):
    """The oracle as it stands on the same synthetic inputs: per shape,
    quantise + double-quantise + dequantise W, then the fp64 forward and
    backward to the input over all 2048 tokens and the LoRA gradients;
    fwd + bwd repeated until about 12 s of CPU time in all (never past
    30 s).  Reported as the fwd + bwd TFLOP/s over the fwd + bwd time."""
    from bit_nf4_quantized_22_amd import synth
    from oracle import linear, nf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    f64 = lambda a: synth.bf16_to_f32(a).astype(np.float64)  # noqa: E731
    t_all = time.perf_counter()
    prepared = []
    for (N, K), wl in workloads:
        w32 = synth.bf16_to_f32(wl.W)
        packed, absmax = nf4.quantize_nf4(w32)
        q8, c2 = nf4.double_quantize(absmax)
        what = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w32.size).reshape(N, K)
        prepared.append((N, K, what.astype(np.float64), f64(wl.x), f64(wl.A), f64(wl.B),
                         f64(wl.dy), wl))
    flops, t_gemm, reps = 0.0, 0.0, 0
    while True:
        for (N, K, what, x, A, B, dy, wl) in prepared:
            t0 = time.perf_counter()
            linear.linear_forward(x, what, A, B, wl.alpha, wl.r)
            linear.linear_backward_input(dy, what, A, B, wl.alpha, wl.r)
            t_gemm += time.perf_counter() - t0
            flops += 2 * linear_flops(N, K, M_TRAIN, RANK)
            if reps == 0:
                linear.lora_grads(x, dy, A, B, wl.alpha, wl.r)
        reps += 1
        # about 12 s of CPU work in all; the next repeat must not pass 30 s
        elapsed = time.perf_counter() - t_all
        if elapsed >= 12.0 or elapsed + t_gemm / reps > 30.0 or reps >= 64:
            break
    # HBM-bound rows on the decode-shaped weight W 4096x11008 (the metric's
    # shape): quantise + double-quantise, dequantise, and the decode forward
    # at M = 1 (dequantise, then the fp64 product with the LoRA term), each
    # once; the quantiser is plain NumPy, which runs on one thread
    (N, K), wl = workloads[1]
    w32 = synth.bf16_to_f32(wl.W)
    t0 = time.perf_counter()
    packed, absmax = nf4.quantize_nf4(w32)
    q8, c2 = nf4.double_quantize(absmax)
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    what = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w32.size).reshape(N, K)
    t_dq = time.perf_counter() - t0
    t0 = time.perf_counter()
    what = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w32.size).reshape(N, K)
    linear.linear_forward(f64(wl.x)[:1], what.astype(np.float64), f64(wl.A), f64(wl.B),
                          wl.alpha, wl.r)
    t_gv = time.perf_counter() - t0
    nk = N * K
    q_rate = nk / t_q
    w65 = Q65_LAYERS * sum(n * k for (_, n, k) in synth.LLAMA65B_TARGETS)
    total = time.perf_counter() - t_all
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                         model)
    except OSError:
        pass
    return {"value": round(flops / t_gemm / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "quantise_GBps": round(nk * (2.5 + 9 / 64) / t_q / 1e9, 4),
            "quantise_s_4096x11008_one_thread": round(t_q, 3),
            "dequant_GBps": round(nk * (BYTES_PER_WEIGHT + 2) / t_dq / 1e9, 4),
            "gemv_GBps": round(gemv_bytes(N, K, 1, RANK) / t_gv / 1e9, 4),
            "gemv_s_per_call_M1": round(t_gv, 3),
            "quantise_65b_80_layers_s_extrapolated": round(w65 / q_rate, 1),
            "quantise_65b_note": f"{w65} weights (80 layers x 7 projections of the 65B "
                                 f"shapes) at the measured one-thread rate of "
                                 f"{q_rate / 1e6:.1f} M weights/s",
            "sample": "oracle on the bench's own inputs: quantise+DQ+dequant of W 11008x4096 and "
                      "4096x11008, fp64 fwd+bwd_dx over all 2048 tokens (r=16) repeated "
                      f"{reps}x, LoRA grads once; quantise+DQ, dequant and one M=1 decode "
                      f"forward of W 4096x11008 once each; {total:.1f} s wall, fwd+bwd "
                      f"{t_gemm:.1f} s; "
                      f"cpu_count={os.cpu_count()}, BLAS threads {threads}, {model}"}


def unfused_context(qn, torch, layers, reps=10):
    """Context, not the metric: the same base products done the unfused way,
    nf4_dequant of W to bf16 in HBM followed by torch's bf16 GEMM (hipBLASLt)
    for y = x W^T and dx = dy W, without the LoRA terms.  Reports the plain
    bf16 GEMM rate (the achievable MFMA rate of a library GEMM at these
    shapes) and the rate of dequant + GEMM."""
    F = torch.nn.functional
    res = {}
    for L in layers:
        qw, N, K = L["qw"], L["N"], L["K"]
        flops = 2.0 * M_TRAIN * N * K
        for name, gemm in (("fwd", lambda: F.linear(L["x"], L["deq"])),
                           ("bwd", lambda: torch.mm(L["dy"], L["deq"]))):
            def run(with_dequant):
                if with_dequant:
                    qn.nf4_dequant(qw, torch.bfloat16, out=L["deq"])
                return gemm()
            for _ in range(3):
                run(True)
            torch.cuda.synchronize()
            t = {}
            for wd in (False, True):
                s = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                s.record()
                for _ in range(reps):
                    run(wd)
                e.record()
                torch.cuda.synchronize()
                t[wd] = s.elapsed_time(e) / reps
            res[f"{name} {N}x{K}"] = {"gemm_us": round(t[False] * 1e3, 1),
                                      "gemm_TFLOPs": round(flops / (t[False] * 1e-3) / 1e12, 1),
                                      "dequant_plus_gemm_us": round(t[True] * 1e3, 1),
                                      "dequant_plus_gemm_TFLOPs":
                                          round(flops / (t[True] * 1e-3) / 1e12, 1)}
    return res


def adamw_7b_lora(qn, torch, dev, synth, steps=10):
    """AdamW step over every LoRA parameter of a 7B model at r = 16 (A and B
    of the seven projections of 32 layers, one flat fp32 buffer each for p,
    g, m, v, plus the bf16 copy of p): HBM-bound, 30 bytes per parameter."""
    n = 32 * sum(RANK * (nn + kk) for (_, nn, kk) in synth.LLAMA7B_TARGETS)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    p = torch.randn(n, generator=gen, device=dev) * 0.01
    g = torch.randn(n, generator=gen, device=dev) * 1e-3
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    qn.lora_adamw_step(p, g, m, v, 1, weight_decay=0.01, p_bf16=pb)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for t in range(2, steps + 2):
        qn.lora_adamw_step(p, g, m, v, t, weight_decay=0.01, p_bf16=pb)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    gbps = n * 30 / (ms * 1e-3) / 1e9
    del p, g, m, v, pb
    torch.cuda.empty_cache()
    return {"params": n, "ms_per_step": round(ms, 4), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}


def dropout_cost(qn, torch, layers, reps=10, p=0.05, seed=7):
    """lora_dropout GB/s and the time the dropout variants add to fwd + bwd."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    xd = [torch.empty_like(L["x"]) for L in layers]

    def drop():
        for L, o in zip(layers, xd):
            qn.lora_dropout(L["x"], p, seed, out=o)

    def plain():
        for L in layers:
            qn.qlora_linear_fwd(L["qw"], L["x"], L["A"], L["B"], RANK, ALPHA, y=L["y"],
                                u_out=L["u"], ws=L["ws"])
            qn.qlora_linear_bwd_dx(L["qw"], L["dy"], L["A"], L["B"], RANK, ALPHA, dx=L["dx"],
                                   t_out=L["t"], ws=L["ws"])

    def dropped():
        for L, o in zip(layers, xd):
            qn.qlora_linear_fwd_dropout(L["qw"], L["x"], o, L["A"], L["B"], RANK, ALPHA,
                                        y=L["y"], u_out=L["u"], ws=L["ws"])
            qn.qlora_linear_bwd_dx_dropout(L["qw"], L["dy"], L["A"], L["B"], RANK, ALPHA, p, seed,
                                           dx=L["dx"], t_out=L["t"], ws=L["ws"])

    # interleaved rounds, medians: the clock drifts between back-to-back runs
    rounds = [(timed(drop), timed(plain), timed(dropped)) for _ in range(5)]
    ms_drop, ms_plain, ms_dropped = (float(np.median([r[i] for r in rounds])) for i in range(3))
    nbytes = sum(2 * 2 * M_TRAIN * L["K"] for L in layers)
    gbps = nbytes / (ms_drop * 1e-3) / 1e9
    return {"p": p, "lora_dropout_ms": round(ms_drop, 4), "lora_dropout_GBps": round(gbps, 1),
            "lora_dropout_frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
            "fwd_bwd_ms": round(ms_plain, 4), "fwd_bwd_dropout_ms": round(ms_dropped, 4),
            "added_ms_incl_lora_dropout": round(ms_dropped + ms_drop - ms_plain, 4)}


def decoder_layer(qn, torch, dev, targets, M, r, alpha, std, seed, with_quantise, reps=5):
    """One decoder layer's seven projections on the device: bf16 N(0, std)
    weights and N(0, 1) activations from torch's generator (seed), A, B
    N(0, 0.01).  Phases (each over all seven, median of reps after a
    warm-up): quantise (quantise + DQ of all seven weights in one
    nf4_quantize_dq_batch launch), fwd, bwd_dx and, with with_quantise,
    lora_grads on the saved u and t."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bf = torch.bfloat16
    projs, acts = [], {}
    for (name, n, k) in targets:
        W = (torch.randn(n, k, generator=gen, device=dev) * std).to(bf)
        qw = qn.quantize_weight(W)
        P = dict(name=name, N=n, K=k, qw=qw,
                 A=(torch.randn(r, k, generator=gen, device=dev) * 0.01).to(bf),
                 B=(torch.randn(n, r, generator=gen, device=dev) * 0.01).to(bf),
                 u=torch.empty((M, r), dtype=bf, device=dev),
                 t=torch.empty((M, r), dtype=bf, device=dev),
                 dA=torch.empty((r, k), device=dev), dB=torch.empty((n, r), device=dev))
        P["W"] = W if with_quantise else None
        for key, dim in (("x", k), ("dy", n), ("y", n), ("dx", k)):
            if (key, dim) not in acts:
                acts[(key, dim)] = torch.randn(M, dim, generator=gen, device=dev).to(bf)
            P[key] = acts[(key, dim)]
        projs.append(P)
    ws = qn.workspace(max(qn.qn_workspace_bytes(op, M, P["N"], P["K"], r)
                          for P in projs for op in (0, 1, 2)), dev)
    torch.cuda.synchronize()

    def run(ph):
        if ph == "quantise":  # the layer's seven weights in one launch
            qn.nf4_quantize_dq_batch([P["W"].reshape(-1) for P in projs],
                                     outs=[(P["qw"].packed, P["qw"].qscale, P["qw"].gscale)
                                           for P in projs])
            return
        for P in projs:
            if ph == "fwd":
                qn.qlora_linear_fwd(P["qw"], P["x"], P["A"], P["B"], r, alpha, y=P["y"],
                                    u_out=P["u"], ws=ws)
            elif ph == "bwd":
                qn.qlora_linear_bwd_dx(P["qw"], P["dy"], P["A"], P["B"], r, alpha, dx=P["dx"],
                                       t_out=P["t"], ws=ws)
            else:
                qn.lora_grads(P["x"], P["dy"], P["A"], P["B"], r, alpha, u=P["u"], t=P["t"],
                              dA=P["dA"], dB=P["dB"], ws=ws)

    phases = (["quantise"] if with_quantise else []) + ["fwd", "bwd"] + \
        (["grads"] if with_quantise else [])
    ms = {}
    for ph in phases:
        run(ph)
        torch.cuda.synchronize()
        # the quantise phase is a single launch: four of them back to back
        # per timing, so the host's preparation of one overlaps the device's
        # work on the previous one instead of being timed
        k = 4 if ph == "quantise" else 1
        ts = []
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(k):
                run(ph)
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e) / k)
        ms[ph] = float(np.median(ts))
    flops = sum(linear_flops(P["N"], P["K"], M, r) for P in projs)
    nk = sum(P["N"] * P["K"] for P in projs)
    res = {"targets": [f"{P['name']} {P['N']}x{P['K']}" for P in projs], "M": M, "r": r,
           "alpha": alpha, "weights": nk, "ms": {k: round(v, 4) for k, v in ms.items()},
           "fwd_TFLOPs": round(flops / (ms["fwd"] * 1e-3) / 1e12, 2),
           "bwd_TFLOPs": round(flops / (ms["bwd"] * 1e-3) / 1e12, 2)}
    res["fwd_bwd_TFLOPs"] = round(2 * flops / ((ms["fwd"] + ms["bwd"]) * 1e-3) / 1e12, 2)
    res["fwd_bwd_frac_mfma"] = round(res["fwd_bwd_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
    if with_quantise:
        qb = nk * (2 + BYTES_PER_WEIGHT)
        res["quantise_GBps"] = round(qb / (ms["quantise"] * 1e-3) / 1e9, 1)
        res["quantise_frac_hbm"] = round(res["quantise_GBps"] / PEAK_HBM_GBPS, 4)
        gb = sum(2 * M * (P["N"] + P["K"]) + 2 * 2 * M * r + 4 * r * (P["N"] + P["K"])
                 for P in projs)
        res["grads_GBps"] = round(gb / (ms["grads"] * 1e-3) / 1e9, 1)
        res["grads_frac_hbm"] = round(res["grads_GBps"] / PEAK_HBM_GBPS, 4)
    del projs, acts, ws
    torch.cuda.empty_cache()
    return res


def decode_layer_7b(qn, torch, dev, synth, r=16, alpha=32.0, std=0.02, seed=9, reps=10):
    """One token (M = 1) through the seven projections of a 7B-shaped layer
    (q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008): bf16 N(0,
    std) weights quantised on the device, x N(0, 1), A, B N(0, 0.01), LoRA
    r = 16.  The seven calls of each of enough layer copies to exceed the
    256 MiB Infinity Cache are captured in one HIP graph; the time per layer
    is a replay's time over the copies (median of reps).  "stacked" times the
    same layer as four calls: q|k|v and gate|up each as one call on
    row-stacked weights with stacked adapters (rank 3r and 2r, block-diagonal
    B, alpha scaled so alpha / r is unchanged)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bf = torch.bfloat16
    targets = synth.LLAMA7B_TARGETS
    layer_bytes = sum(n * k for _, n, k in targets) * BYTES_PER_WEIGHT
    ncopy = int(np.ceil(ROTATE_BYTES / layer_bytes))
    Ws = {(n, k): (torch.randn(n, k, generator=gen, device=dev) * std).to(bf) for _, n, k in targets}
    copies = [[qn.quantize_weight(Ws[(n, k)]) for _, n, k in targets] for _ in range(ncopy)]
    xs = {k: torch.randn(1, k, generator=gen, device=dev).to(bf) for _, _, k in targets}
    ys = [torch.empty((1, n), dtype=bf, device=dev) for _, n, _ in targets]
    ada = [((torch.randn(r, k, generator=gen, device=dev) * 0.01).to(bf),
            (torch.randn(n, r, generator=gen, device=dev) * 0.01).to(bf)) for _, n, k in targets]
    ws = qn.workspace(max(qn.qn_workspace_bytes(0, 1, n, k, r) for _, n, k in targets), dev)

    def calls():
        for layer in copies:
            for t, ((name, n, k), qw, (A, B)) in enumerate(zip(targets, layer, ada)):
                qn.qlora_linear_fwd(qw, xs[k], A, B, r, alpha, y=ys[t], ws=ws)

    # Projections that read the same input as one call on row-stacked
    # weights: q|k|v ([12288, 4096], adapters stacked to rank 3r with a
    # block-diagonal B and alpha scaled by 3, so alpha / r is unchanged) and
    # gate|up ([22016, 4096], rank 2r); o and down as before.  Quantising the
    # stack gives the separate codes and constants byte for byte.
    def stack_adapters(idx):
        A = torch.cat([ada[i][0] for i in idx])
        n = sum(targets[i][1] for i in idx)
        B = torch.zeros((n, r * len(idx)), dtype=bf, device=dev)
        row = 0
        for j, i in enumerate(idx):
            B[row:row + targets[i][1], j * r:(j + 1) * r] = ada[i][1]
            row += targets[i][1]
        return A, B
    fused = [([0, 1, 2], stack_adapters([0, 1, 2])), ([3], ada[3]),
             ([4, 5], stack_adapters([4, 5])), ([6], ada[6])]
    Wcat = {}
    for idx, _ in fused:
        Wcat[tuple(idx)] = torch.cat([Ws[(targets[i][1], targets[i][2])] for i in idx])
    fcopies = [[qn.quantize_weight(Wcat[tuple(idx)]) for idx, _ in fused] for _ in range(ncopy)]
    del Wcat, Ws
    ys_f = [torch.empty((1, sum(targets[i][1] for i in idx)), dtype=bf, device=dev)
            for idx, _ in fused]
    ws_f = qn.workspace(max(qn.qn_workspace_bytes(0, 1, y.shape[1], targets[idx[0]][2],
                                                  r * len(idx))
                            for (idx, _), y in zip(fused, ys_f)), dev)

    def calls_fused():
        for layer in fcopies:
            for qw, (idx, (A, B)), y in zip(layer, fused, ys_f):
                qn.qlora_linear_fwd(qw, xs[targets[idx[0]][2]], A, B, r * len(idx),
                                    alpha * len(idx), y=y, ws=ws_f)

    def graph_of(fn):
        stream = torch.cuda.current_stream()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            fn()  # eager warm-up on the capture stream
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                fn()
        stream.wait_stream(gs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    def time_replays(g):
        ts = []
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            g.replay()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return float(np.median(ts)) * 1e3 / ncopy

    g = graph_of(calls)
    us = time_replays(g)
    gf = graph_of(calls_fused)
    us_f = time_replays(gf)
    # the last copy's outputs, stacked call against separate calls
    diff = 0.0
    for (idx, _), y in zip(fused, ys_f):
        col = 0
        for i in idx:
            n_i = targets[i][1]
            a, b = y[0, col:col + n_i].float(), ys[i][0].float()
            diff = max(diff, float((a - b).norm() / b.norm()))
            col += n_i
    nbytes = layer_bytes + sum(2 * (n + k) + 2 * r * (n + k) for _, n, k in targets)
    res = {"targets": [f"{name} {n}x{k}" for name, n, k in targets], "M": 1, "r": r,
           "alpha": alpha, "layer_copies": ncopy, "us_per_layer": round(us, 3),
           "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
           "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
           "ms_per_token_32_layers": round(32 * us / 1e3, 4),
           "stacked": {"us_per_layer": round(us_f, 3),
                       "GBps": round(nbytes / (us_f * 1e-6) / 1e9, 1),
                       "frac_hbm": round(nbytes / (us_f * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                       "ms_per_token_32_layers": round(32 * us_f / 1e3, 4),
                       "max_rel_diff_vs_separate": round(diff, 6),
                       "calls": "q|k|v stacked (rank 3r, block-diagonal B), o, gate|up "
                                "stacked (rank 2r), down: four calls per layer"},
           "note": "the seven linear layers only (no attention, norms or sampling)"}
    del g, gf, copies, fcopies, xs, ys, ys_f, ada, fused, ws, ws_f
    torch.cuda.empty_cache()
    return res


def hbm_peak(qn, torch, dev, reps=10):
    """Achievable HBM rates measured with plain torch kernels on 1 GiB
    buffers (context for the fractions of the 8 TB/s peak): a device copy
    (read + write) and a float32 sum (read only)."""
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    nbytes = a.numel() * 4

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t_copy = timed(lambda: b.copy_(a))
    t_read = timed(lambda: a.sum())
    t_probe = timed(lambda: qn.hbm_read_probe(a, sink))
    del a, b
    torch.cuda.empty_cache()
    return {"read_probe_GBps": round(nbytes / (t_probe * 1e-3) / 1e9, 1),
            "copy_GBps": round(2 * nbytes / (t_copy * 1e-3) / 1e9, 1),
            "read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "buffer_bytes": nbytes,
            "kernels": "qn_hbm_read_probe (16-byte streaming loads, read only), torch copy_ "
                       "(read + write) and torch sum of fp32 (read), 1 GiB each"}


def quantise_65b(qn, torch, dev, synth):
    """Quantiser throughput over Q65_LAYERS layers of the 65B shapes."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    layers = []
    for _ in range(Q65_DISTINCT):
        proj = []
        for (_, n, k) in synth.LLAMA65B_TARGETS:
            w = (torch.randn(n * k, generator=gen, device=dev) * 0.015).to(torch.bfloat16)
            proj.append((w, torch.empty(n * k // 2, dtype=torch.uint8, device=dev),
                         torch.empty(n * k // 64, dtype=torch.uint8, device=dev),
                         torch.empty(-(-n * k // (64 * 256)), dtype=torch.float32, device=dev)))
        layers.append(proj)
    numel = sum(n * k for (_, n, k) in synth.LLAMA65B_TARGETS)

    def run():  # one nf4_quantize_dq_batch launch per layer (its seven weights)
        for i in range(Q65_LAYERS):
            proj = layers[i % Q65_DISTINCT]
            qn.nf4_quantize_dq_batch([w for (w, _, _, _) in proj],
                                     outs=[(packed, q8, c2) for (_, packed, q8, c2) in proj])

    run()  # warm-up
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    # read bf16 W, write the codes, q8 and c2
    nbytes = Q65_LAYERS * numel * (2 + BYTES_PER_WEIGHT)
    gbps = nbytes / (ms * 1e-3) / 1e9
    del layers
    torch.cuda.empty_cache()
    return {"layers": Q65_LAYERS, "distinct_layers": Q65_DISTINCT,
            "weights_per_layer": numel, "ms": round(ms, 3),
            "ms_per_layer": round(ms / Q65_LAYERS, 4),
            "weights_per_s": round(Q65_LAYERS * numel / (ms * 1e-3), 1),
            "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(how the path would shard across GPUs is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_nf4_quantized_22_amd as qn
    from bit_nf4_quantized_22_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    layers, workloads = [], []
    for (N, K) in SHAPES:
        wl = synth.train_linear(N, K, M=M_TRAIN, seed=3, r=RANK, alpha=ALPHA)
        workloads.append(((N, K), wl))
        L = dict(N=N, K=K, W=bf(wl.W).reshape(N, K), x=bf(wl.x), A=bf(wl.A), B=bf(wl.B),
                 dy=bf(wl.dy))
        L["qw"] = qn.quantize_weight(L["W"])
        L["deq"] = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        L["y"] = torch.empty((M_TRAIN, N), dtype=torch.bfloat16, device=dev)
        L["dx"] = torch.empty((M_TRAIN, K), dtype=torch.bfloat16, device=dev)
        L["u"] = torch.empty((M_TRAIN, RANK), dtype=torch.bfloat16, device=dev)
        L["t"] = torch.empty((M_TRAIN, RANK), dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty((RANK, K), dtype=torch.float32, device=dev)
        L["dB"] = torch.empty((N, RANK), dtype=torch.float32, device=dev)
        ws_b = max(qn.qn_workspace_bytes(op, M_TRAIN, N, K, RANK) for op in (0, 1, 2, 3))
        L["ws"] = qn.workspace(ws_b, dev)
        # decode: distinct quantised copies (Infinity Cache defeat), own workspace
        ncopy = int(np.ceil(ROTATE_BYTES / (N * K * BYTES_PER_WEIGHT)))
        L["copies"] = [qn.quantize_weight(L["W"]) for _ in range(ncopy)]
        L["ydec"] = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in DECODE_M}
        L["wsdec"] = qn.workspace(qn.qn_workspace_bytes(0, max(DECODE_M), N, K, RANK), dev)
        layers.append(L)
    torch.cuda.synchronize()

    # the q_proj decode shape: W 4096x4096 N(0, 0.02), its own x, A, B
    sq = synth.decode_layer(max(DECODE_M), *DECODE_SQUARE, seed=2, r=RANK, alpha=ALPHA)
    Lsq = dict(N=sq.N, K=sq.K, W=bf(sq.W).reshape(sq.N, sq.K), x=bf(sq.x), A=bf(sq.A),
               B=bf(sq.B))
    ncopy = int(np.ceil(ROTATE_BYTES / (sq.N * sq.K * BYTES_PER_WEIGHT)))
    Lsq["copies"] = [qn.quantize_weight(Lsq["W"]) for _ in range(ncopy)]
    Lsq["ydec"] = {m: torch.empty((m, sq.N), dtype=torch.bfloat16, device=dev) for m in DECODE_M}
    Lsq["wsdec"] = qn.workspace(qn.qn_workspace_bytes(0, max(DECODE_M), sq.N, sq.K, RANK), dev)
    torch.cuda.synchronize()

    # decode graphs: one per (shape, M), each call on the next copy
    stream = torch.cuda.current_stream()
    graphs = {}
    # (N, K, M, r): the decode calls with the LoRA term, and at M = 1 also
    # without it (r = 0: the GEMV kernel is the whole call)
    for L in layers + [Lsq]:
        for m, r in [(m, RANK) for m in DECODE_M] + [(1, 0)]:
            def calls(L=L, m=m, r=r):
                for c in L["copies"]:
                    qn.qlora_linear_fwd(c, L["x"][:m], L["A"] if r else None,
                                        L["B"] if r else None, r, ALPHA,
                                        y=L["ydec"][m], ws=L["wsdec"])
            gs = torch.cuda.Stream()
            gs.wait_stream(stream)
            with torch.cuda.stream(gs):
                calls()  # eager warm-up on the capture stream
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=gs):
                    calls()
            stream.wait_stream(gs)
            graphs[(L["N"], L["K"], m, r)] = (g, len(L["copies"]))
    torch.cuda.synchronize()

    phases = ["quantise", "dequant", "gemm", "fwd", "bwd", "grads", "merge", "gemv"]

    def step(record):
        ev = {}
        for ph in phases:
            if ph == "gemv":
                for key, (g, n) in graphs.items():
                    s = torch.cuda.Event(enable_timing=True)
                    e = torch.cuda.Event(enable_timing=True)
                    s.record()
                    g.replay()
                    e.record()
                    ev[("gemv",) + key] = (s, e)
                continue
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            if ph == "quantise":  # both weights in one launch
                qn.nf4_quantize_dq_batch([L["W"].reshape(-1) for L in layers],
                                         outs=[(L["qw"].packed, L["qw"].qscale, L["qw"].gscale)
                                               for L in layers])
            for L in layers:
                qw = L["qw"]
                if ph == "quantise":
                    break
                elif ph == "dequant":
                    qn.nf4_dequant(qw, torch.bfloat16, out=L["deq"])
                elif ph == "gemm":
                    qn.qlora_linear_fwd(qw, L["x"], None, None, 0, ALPHA, y=L["y"])
                elif ph == "fwd":
                    qn.qlora_linear_fwd(qw, L["x"], L["A"], L["B"], RANK, ALPHA, y=L["y"],
                                        u_out=L["u"], ws=L["ws"])
                elif ph == "bwd":
                    qn.qlora_linear_bwd_dx(qw, L["dy"], L["A"], L["B"], RANK, ALPHA, dx=L["dx"],
                                           t_out=L["t"], ws=L["ws"])
                elif ph == "merge":
                    qn.qlora_merge(qw, L["A"], L["B"], RANK, ALPHA, out=L["deq"])
                elif ph == "grads":
                    qn.lora_grads(L["x"], L["dy"], L["A"], L["B"], RANK, ALPHA, u=L["u"],
                                  t=L["t"], dA=L["dA"], dB=L["dB"], ws=L["ws"])
            e.record()
            ev[ph] = (s, e)
        if record is not None:
            record.append(ev)

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(recs)
        print(f"step {i + 1}/{args.steps}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def mean_ms(key):
        return float(np.mean([r[key][0].elapsed_time(r[key][1]) for r in recs]))

    ms = {ph: mean_ms(ph) for ph in phases if ph != "gemv"}
    spread = {ph: [round(float(np.percentile([r[ph][0].elapsed_time(r[ph][1]) for r in recs], q)), 4)
                   for q in (10, 50, 90)] for ph in phases if ph != "gemv"}
    gemv = {}
    gemv_ms_total = 0.0
    for key, (g, n) in graphs.items():
        t = mean_ms(("gemv",) + key)
        gemv_ms_total += t
        N, K, m, r = key
        us = t * 1e3 / n
        gbps = gemv_bytes(N, K, m, r) / (us * 1e-6) / 1e9
        gemv[f"{N}x{K}_M{m}" + ("" if r else "_r0")] = {
            "us_per_call": round(us, 3), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
    ms["gemv"] = gemv_ms_total
    step_ms = wall / args.steps * 1e3

    fwd_flops = sum(linear_flops(L["N"], L["K"], M_TRAIN, RANK) for L in layers)
    gemm_flops = sum(2 * M_TRAIN * L["N"] * L["K"] for L in layers)  # r = 0 calls
    gemm_tflops = 2 * fwd_flops / ((ms["fwd"] + ms["bwd"]) * 1e-3) / 1e12
    # quantise + DQ in one launch: read bf16 W, write the codes, q8 and c2
    q_bytes = sum(L["N"] * L["K"] * (2 + BYTES_PER_WEIGHT) for L in layers)
    dq_bytes = sum(L["N"] * L["K"] * (BYTES_PER_WEIGHT + 2) for L in layers)
    # grads: read x, dy (bf16) and the saved u, t (bf16); write dA, dB (fp32)
    gr_bytes = sum(2 * M_TRAIN * (L["N"] + L["K"]) + 2 * 2 * M_TRAIN * RANK
                   + 4 * RANK * (L["N"] + L["K"]) for L in layers)
    # merge: read codes + constants, A and B; write the bf16 weight
    mg_bytes = sum(L["N"] * L["K"] * (BYTES_PER_WEIGHT + 2) + 2 * RANK * (L["N"] + L["K"])
                   for L in layers)
    hN, hK, hM = GEMV_HEADLINE
    head = gemv[f"{hN}x{hK}_M{hM}"]
    per_phase = {
        "quantise": ("hbm", q_bytes / (ms["quantise"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "dequant": ("hbm", dq_bytes / (ms["dequant"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "gemm": ("mfma", gemm_flops / (ms["gemm"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "fwd": ("mfma", fwd_flops / (ms["fwd"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "bwd": ("mfma", fwd_flops / (ms["bwd"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "grads": ("hbm", gr_bytes / (ms["grads"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "merge": ("hbm", mg_bytes / (ms["merge"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "gemv": ("hbm", head["GBps"], PEAK_HBM_GBPS, "GB/s"),
    }
    # dominant kernel: the fused dequant GEMM, one launch per "gemm" call
    # (both shapes: average flops per launch over average launch time)
    launches = len(layers)
    gemm_us_per_launch = ms["gemm"] * 1e3 / launches
    achieved = gemm_flops / launches / (gemm_us_per_launch * 1e-6) / 1e12
    traffic = pmc_traffic()
    out = {
        "metric": METRIC,
        "value": round(gemm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded numpy PCG64; W bf16 Student-t(5) scaled to std 0.02; "
                "x, dy bf16 N(0,1); A, B bf16 N(0,0.01)",
        "config": {"workload": "training-step linear at the 7B MLP shapes, W 11008x4096 and "
                               "4096x11008 NF4+double-quant, M=2048 tokens, LoRA r=16 alpha=32: "
                               "quantise+DQ, dequant, fwd, bwd_dx, lora_grads; plus decode "
                               "(LoRA-down + dequant GEMV) at M=1,4,16 on rotating copies of "
                               "both MLP weights and of W 4096x4096 N(0,0.02)",
                   "M": M_TRAIN, "r": RANK, "alpha": ALPHA,
                   "weights": [f"{n}x{k}" for n, k in SHAPES], "decode_M": list(DECODE_M)},
        "gemv": {"shape": f"{hN}x{hK}", "M": hM, "GBps": head["GBps"],
                 "frac_hbm": head["frac_hbm"], "us_per_call": head["us_per_call"],
                 "kernel_only_r0": gemv[f"{hN}x{hK}_M{hM}_r0"],
                 "all": gemv},
        "phases_ms": {k: round(v, 4) for k, v in ms.items()},
        "phases_ms_p10_p50_p90": spread,
        "phase_rates": {k: {"bound": v[0], "achieved": round(v[1], 2), "unit": v[3],
                            "frac": round(v[1] / v[2], 4)} for k, v in per_phase.items()},
        "roofline": {"kernel": "fused dequant GEMM kernel, one launch (qlora_linear_fwd with r=0), "
                               "M=2048, W 11008x4096 and 4096x11008",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "us_per_launch": round(gemm_us_per_launch, 2)},
    }
    for L in layers + [Lsq]:
        del L["copies"]
    del graphs
    torch.cuda.empty_cache()
    sections = [
        ("layer_7b", lambda: decoder_layer(qn, torch, dev, synth.LLAMA7B_TARGETS,
                                           with_quantise=True, **LAYER7B)),
        ("layer_65b", lambda: decoder_layer(qn, torch, dev, synth.LLAMA65B_TARGETS,
                                            with_quantise=False, **LAYER65B)),
        ("decode_layer_7b", lambda: decode_layer_7b(qn, torch, dev, synth)),
        ("hbm_measured", lambda: hbm_peak(qn, torch, dev)),
        ("unfused_context", lambda: unfused_context(qn, torch, layers)),
        ("quantise_65b", lambda: quantise_65b(qn, torch, dev, synth)),
        ("adamw_7b_lora", lambda: adamw_7b_lora(qn, torch, dev, synth)),
        ("dropout", lambda: dropout_cost(qn, torch, layers)),
    ]
    if not args.no_cpu_baseline:
        sections.append(("cpu_baseline", lambda: cpu_baseline(workloads)))
    for name, run in sections:
        out[name] = run()
        print(f"{name} done", file=sys.stderr, flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
