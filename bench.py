#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step = one pass of the whole hot path over the training-step linear
workload at the 7B MLP shapes, for both orientations of the weight
(gate/up W 11008x4096 and down W 4096x11008, bf16 Student-t(5) weights
scaled to std 0.02, M = 2048 tokens, LoRA r = 16, alpha = 32):
  quantise  nf4_quantize + dq_quantize_scales of the bf16 weight
  dequant   nf4_dequant to bf16 (the standalone bit-exact expansion)
  fwd       qlora_linear_fwd   at M = 2048 (u = x A^T + fused dequant GEMM)
  bwd       qlora_linear_bwd_dx at M = 2048 (t = dy B + fused dequant GEMM)
  grads     lora_grads with the saved u, t
  gemv      qlora_linear_fwd at M = 1, 4, 16 (decode), rotating over
            >= 512 MB of distinct quantised copies so no call is served
            from the 256 MB Infinity Cache.
Inputs are resident in HBM before the timed region.  Every phase is timed
with HIP events on the stream the library launches on (torch's current
stream).

Printed JSON line: value = dequant-GEMM TFLOP/s (2MNK + LoRA flops of the
fwd and bwd calls over their event time); the decode GEMV GB/s and its
fraction of HBM peak sit in "gemv"; "roofline" is the phase with the largest
share of the step time.
"""

import argparse
import json
import os
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
ROTATE_BYTES = 512 << 20

BYTES_PER_WEIGHT = 0.5 + 1 / 64 + 4 / (64 * 256)  # NF4 codes + q8 + c2


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one plain 256 MiB device copy (counter calibration)")
    return p.parse_args()


def gemv_bytes(N, K, M, r):
    return N * K * BYTES_PER_WEIGHT + 2 * r * (N + K) + 2 * M * (K + N) + 2 * M * r


def linear_flops(N, K, M, r):
    return 2.0 * M * N * K + 2.0 * M * r * (N + K)


def cpu_baseline():
    """The oracle as it stands, on a bounded sample of the same workload:
    quantise + double-quantise + dequantise W 4096x11008 and the fp64
    forward of 256 of the 2048 tokens.  Reported as TFLOP/s of the forward
    (2 M N K + LoRA flops over the whole sample's time)."""
    from bit_nf4_quantized_22_amd import synth
    from oracle import linear, nf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    N, K = 4096, 11008
    wl = synth.train_linear(N, K, M=256, seed=3)
    t0 = time.perf_counter()
    w32 = synth.bf16_to_f32(wl.W)
    packed, absmax = nf4.quantize_nf4(w32)
    q8, c2 = nf4.double_quantize(absmax)
    What = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w32.size).reshape(N, K)
    x = synth.bf16_to_f32(wl.x).astype(np.float64)
    A = synth.bf16_to_f32(wl.A).astype(np.float64)
    B = synth.bf16_to_f32(wl.B).astype(np.float64)
    linear.linear_forward(x, What.astype(np.float64), A, B, wl.alpha, wl.r)
    dt = time.perf_counter() - t0
    flops = linear_flops(N, K, 256, RANK)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "oracle quantise+DQ+dequant of W 4096x11008 and fp64 forward of 256 of "
                      f"2048 tokens (r=16), {dt:.1f} s wall; cpu_count={os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU data-parallel layout is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_nf4_quantized_22_amd as qn
    from bit_nf4_quantized_22_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    layers = []
    for (N, K) in SHAPES:
        wl = synth.train_linear(N, K, M=M_TRAIN, seed=3, r=RANK, alpha=ALPHA)
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
        ws_b = max(qn.qn_workspace_bytes(op, M_TRAIN, N, K, RANK) for op in (0, 1, 2))
        L["ws"] = torch.empty(ws_b, dtype=torch.uint8, device=dev)
        # distinct quantised copies for the decode GEMV (Infinity Cache defeat)
        ncopy = int(np.ceil(ROTATE_BYTES / (N * K * BYTES_PER_WEIGHT)))
        L["copies"] = [qn.quantize_weight(L["W"]) for _ in range(ncopy)]
        L["ydec"] = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in DECODE_M}
        layers.append(L)
    torch.cuda.synchronize()

    phases = ["quantise", "dequant", "fwd", "bwd", "grads", "gemv"]
    rot = [0]

    def step(record):
        ev = {}
        for ph in phases:
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for L in layers:
                qw = L["qw"]
                if ph == "quantise":
                    qn.nf4_quantize(L["W"].reshape(-1), qw.packed, L["absmax_buf"])
                    qn.dq_quantize_scales(L["absmax_buf"], qw.qscale, qw.gscale)
                elif ph == "dequant":
                    qn.nf4_dequant(qw, torch.bfloat16, out=L["deq"])
                elif ph == "fwd":
                    qn.qlora_linear_fwd(qw, L["x"], L["A"], L["B"], RANK, ALPHA, y=L["y"],
                                        u_out=L["u"], ws=L["ws"])
                elif ph == "bwd":
                    qn.qlora_linear_bwd_dx(qw, L["dy"], L["A"], L["B"], RANK, ALPHA, dx=L["dx"],
                                           t_out=L["t"], ws=L["ws"])
                elif ph == "grads":
                    qn.lora_grads(L["x"], L["dy"], L["A"], L["B"], RANK, ALPHA, u=L["u"],
                                  t=L["t"], dA=L["dA"], dB=L["dB"], ws=L["ws"])
                else:
                    for m in DECODE_M:
                        c = L["copies"][rot[0] % len(L["copies"])]
                        rot[0] += 1
                        qn.qlora_linear_fwd(c, L["x"][:m], L["A"], L["B"], RANK, ALPHA,
                                            y=L["ydec"][m], ws=L["ws"])
            e.record()
            ev[ph] = (s, e)
        if record is not None:
            record.append(ev)

    for L in layers:
        L["absmax_buf"] = torch.empty(L["N"] * L["K"] // 64, dtype=torch.float32, device=dev)

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
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

    ms = {ph: float(np.mean([r[ph][0].elapsed_time(r[ph][1]) for r in recs])) for ph in phases}
    step_ms = sum(ms.values())
    gemm_flops = sum(2 * linear_flops(L["N"], L["K"], M_TRAIN, RANK) for L in layers)
    gemm_tflops = gemm_flops / ((ms["fwd"] + ms["bwd"]) * 1e-3) / 1e12
    dec_bytes = sum(gemv_bytes(L["N"], L["K"], m, RANK) for L in layers for m in DECODE_M)
    gemv_gbps = dec_bytes / (ms["gemv"] * 1e-3) / 1e9
    # quantise: read bf16 W, write codes + fp32 absmax; DQ: read absmax, write q8 (+ c2)
    q_bytes = sum(L["N"] * L["K"] * (2 + 0.5) + L["N"] * L["K"] / 64 * (4 + 4 + 1)
                  for L in layers)
    dq_bytes = sum(L["N"] * L["K"] * (BYTES_PER_WEIGHT + 2) for L in layers)
    # grads: read x, dy (bf16) and the saved u, t (bf16); write dA, dB (fp32)
    gr_bytes = sum(2 * M_TRAIN * (L["N"] + L["K"]) + 2 * 2 * M_TRAIN * RANK
                   + 4 * RANK * (L["N"] + L["K"]) for L in layers)
    per_phase = {
        "quantise": ("hbm", q_bytes / (ms["quantise"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "dequant": ("hbm", dq_bytes / (ms["dequant"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "fwd": ("mfma", sum(linear_flops(L["N"], L["K"], M_TRAIN, RANK) for L in layers)
                / (ms["fwd"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "bwd": ("mfma", sum(linear_flops(L["N"], L["K"], M_TRAIN, RANK) for L in layers)
                / (ms["bwd"] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "grads": ("hbm", gr_bytes / (ms["grads"] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"),
        "gemv": ("hbm", gemv_gbps, PEAK_HBM_GBPS, "GB/s"),
    }
    dom = max(phases, key=lambda p: ms[p])
    bound, ach, peak, unit = per_phase[dom]
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
                               "quantise+DQ, dequant, fwd, bwd_dx, lora_grads; plus decode GEMV "
                               "M=1,4,16 on rotating quantised copies",
                   "M": M_TRAIN, "r": RANK, "alpha": ALPHA,
                   "weights": [f"{n}x{k}" for n, k in SHAPES], "decode_M": list(DECODE_M)},
        "gemv": {"GBps": round(gemv_gbps, 1), "frac_hbm": round(gemv_gbps / PEAK_HBM_GBPS, 4),
                 "bytes_per_call_set": int(dec_bytes)},
        "phases_ms": {k: round(v, 4) for k, v in ms.items()},
        "phase_rates": {k: {"bound": v[0], "achieved": round(v[1], 2), "unit": v[3],
                            "frac": round(v[1] / v[2], 4)} for k, v in per_phase.items()},
        "wall_s_timed": round(wall, 3),
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(ach, 2), "peak": peak,
                     "unit": unit, "frac": round(ach / peak, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
