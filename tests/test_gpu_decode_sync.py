"""Decode forward (M <= 16) calls in sequences that a wrong hand-off
between its two launches would show: the skinny kernel writes the fp32
partial sums of u = x A^T to the caller's workspace and the GEMV launch
sums them in its epilogue.  Launches run back to back with different
inputs, shapes, ranks and grid sizes (so a GEMV that read the previous
call's partial sums would be off), on two streams at once (each with its
own workspace), and replayed from a captured graph with new inputs each
time (against the eager call, bit for bit, and the oracle).  A and B are
drawn large enough that the LoRA term is as large as the base product.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import DEV, bf16_dev, check, f64, linear, quantized_layer, synth, to_bits16, to_np

pytestmark = pytest.mark.gpu


def _layer(N, K, r, seed, M=16):
    wl = synth.decode_layer(M, N, K, seed=seed, r=r)
    rng = np.random.default_rng(seed + 100)
    wl["A"] = synth.bf16_bits((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    wl["B"] = synth.bf16_bits((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    qw, ref = quantized_layer(wl)
    return dict(wl=wl, qw=qw, What=ref["What"].astype(np.float64), A=bf16_dev(wl["A"]),
                B=bf16_dev(wl["B"]))


def _x(M, K, seed):
    return synth.bf16_bits(np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32))


def _want(L, x_bits):
    wl = L["wl"]
    return linear.linear_forward(f64(x_bits), L["What"], f64(wl.A), f64(wl.B), wl.alpha, wl.r)


def test_back_to_back_calls_with_changing_inputs_and_grids():
    # (N, K, r): four bands of 16 rows (fewer GEMV waves than u slices),
    # more bands, and a rank-128 layer whose M r exceeds the workgroup's
    # threads
    layers = [_layer(64, 4096, 16, 1), _layer(512, 4096, 16, 2), _layer(256, 2048, 64, 3),
              _layer(512, 1024, 128, 4)]
    calls = [(0, 1), (1, 1), (2, 4), (3, 16), (1, 16), (0, 16), (2, 1), (3, 1), (1, 1), (0, 1)]
    outs = []
    for i, (li, M) in enumerate(calls):  # no synchronisation between the launches
        L = layers[li]
        xb = _x(M, L["wl"].K, 500 + i)
        u = torch.empty((M, L["wl"].r), dtype=torch.bfloat16, device=DEV)
        y = qn.qlora_linear_fwd(L["qw"], bf16_dev(xb), L["A"], L["B"], L["wl"].r, L["wl"].alpha,
                                u_out=u)
        outs.append((L, xb, y, u))
    torch.cuda.synchronize()
    for i, (L, xb, y, u) in enumerate(outs):
        wl = L["wl"]
        check(f"call {i} y N={wl.N} K={wl.K} r={wl.r} M={xb.shape[0]}", to_np(y), _want(L, xb))
        check(f"call {i} u", to_np(u), linear.lora_down(f64(xb), f64(wl.A)))


def test_two_streams_at_once():
    layers = [_layer(1024, 4096, 16, 5), _layer(512, 2048, 32, 6)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(12):
        si = i % 2
        L = layers[si]
        M = [1, 4, 16][i % 3]
        xb = _x(M, L["wl"].K, 700 + i)
        with torch.cuda.stream(streams[si]):
            x = bf16_dev(xb)
            ws = qn.workspace(qn.qn_workspace_bytes(0, M, L["wl"].N, L["wl"].K, L["wl"].r), DEV)
            y = qn.qlora_linear_fwd(L["qw"], x, L["A"], L["B"], L["wl"].r, L["wl"].alpha, ws=ws)
        outs.append((L, xb, y, x, ws))
    torch.cuda.synchronize()
    for i, (L, xb, y, _, _) in enumerate(outs):
        check(f"stream {i % 2} call {i} M={xb.shape[0]}", to_np(y), _want(L, xb))


@pytest.mark.parametrize("M", [1, 16])
def test_graph_replays_with_new_inputs(M):
    L = _layer(1024, 4096, 16, 7)
    wl = L["wl"]
    xs = torch.empty((M, wl.K), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty((M, wl.N), dtype=torch.bfloat16, device=DEV)
    ws = qn.workspace(qn.qn_workspace_bytes(0, M, wl.N, wl.K, wl.r), DEV)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        xs.copy_(bf16_dev(_x(M, wl.K, 900)))
        qn.qlora_linear_fwd(L["qw"], xs, L["A"], L["B"], wl.r, wl.alpha, y=ys, ws=ws)  # warm-up
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            qn.qlora_linear_fwd(L["qw"], xs, L["A"], L["B"], wl.r, wl.alpha, y=ys, ws=ws)
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    for rep in range(4):
        xb = _x(M, wl.K, 901 + rep)
        xs.copy_(bf16_dev(xb))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_bits16(ys)
        eager = qn.qlora_linear_fwd(L["qw"], bf16_dev(xb), L["A"], L["B"], wl.r, wl.alpha)
        torch.cuda.synchronize()
        assert np.array_equal(got, to_bits16(eager)), f"replay {rep} differs from the eager call"
        check(f"graph replay {rep} M={M}", to_np(ys), _want(L, xb))
