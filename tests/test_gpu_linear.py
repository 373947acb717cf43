"""Parity of the QLoRA linear layer (forward, backward to the input, LoRA
gradients) with the fp64 CPU oracle (GPU).

Bar: relative Frobenius error <= 1e-2 per output (bf16 operands, fp32
accumulation).  The oracle multiplies the exact fp32 dequantised weight in
fp64; the HIP path rounds it to bf16 for the MFMA, so the expected error is
the bf16 rounding of weights, activations and outputs (~1e-3).
"""

import functools

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import (TOL, bf16_dev, check, f32_dev, f64, linear, nf4, quantized_layer,
                               rel_frob, run_layer_checks, synth, to_bits16, to_np)

pytestmark = pytest.mark.gpu


_layer = quantized_layer
_check = check
_run_all = run_layer_checks


@pytest.mark.parametrize("M", [1, 16, 17, 33, 200])
def test_tiny_layer_all_outputs(M):
    wl = synth.tiny_layer(0)
    if M > wl.M:  # extend x, dy with more seeded rows
        rng = np.random.default_rng(1000 + M)
        wl["x"] = synth.bf16_bits(rng.standard_normal((M, wl.K)).astype(np.float32))
        wl["dy"] = synth.bf16_bits(rng.standard_normal((M, wl.N)).astype(np.float32))
    _run_all(wl, M=M)


def test_tiny_layer_without_double_quant():
    _run_all(synth.tiny_layer(0), double_quant=False)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_gemv_4096(M):
    wl = synth.decode_layer(M, 4096, 4096, seed=2)
    qw, ref = _layer(wl)
    x, A, B = bf16_dev(wl.x), bf16_dev(wl.A), bf16_dev(wl.B)
    y = qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha)
    torch.cuda.synchronize()
    want = linear.linear_forward(f64(wl.x), ref["What"].astype(np.float64), f64(wl.A), f64(wl.B),
                                 wl.alpha, wl.r)
    _check(f"y M={M}", to_np(y), want)


@pytest.mark.parametrize("M", [1, 5, 16])
def test_decode_gemv_rank64(M):
    # r = 64, alpha = 16 (the largest LoRA setting the tests use) on the decode path
    wl = synth.decode_layer(M, 4096, 4096, seed=2, r=64, alpha=16.0)
    qw, ref = _layer(wl)
    u = torch.empty((M, wl.r), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw, bf16_dev(wl.x), bf16_dev(wl.A), bf16_dev(wl.B), wl.r, wl.alpha,
                            u_out=u)
    torch.cuda.synchronize()
    want = linear.linear_forward(f64(wl.x), ref["What"].astype(np.float64), f64(wl.A), f64(wl.B),
                                 wl.alpha, wl.r)
    _check(f"y r=64 M={M}", to_np(y), want)
    _check(f"u r=64 M={M}", to_np(u), linear.lora_down(f64(wl.x), f64(wl.A)))


@pytest.mark.parametrize("shape", [(4096, 11008), (11008, 4096)])
@pytest.mark.parametrize("M", [1, 16])
def test_decode_gemv_llama_mlp_shapes(shape, M):
    wl = synth.decode_layer(M, *shape, seed=2)
    qw, ref = _layer(wl)
    y = qn.qlora_linear_fwd(qw, bf16_dev(wl.x), bf16_dev(wl.A), bf16_dev(wl.B), wl.r, wl.alpha)
    torch.cuda.synchronize()
    want = linear.linear_forward(f64(wl.x), ref["What"].astype(np.float64), f64(wl.A), f64(wl.B),
                                 wl.alpha, wl.r)
    _check(f"y {shape} M={M}", to_np(y), want)


@pytest.mark.parametrize("shape", [(11008, 4096), (4096, 11008)])
def test_training_step_linear_full_size(shape):
    # M = 2048 tokens; y and dx checked on 256 sampled rows (each row of y /
    # dx depends only on the same row of x / dy), dA and dB in full.
    wl = synth.train_linear(*shape, M=2048, seed=3)
    rows = np.sort(np.random.default_rng(0).choice(2048, 256, replace=False))
    _run_all(wl, rows=rows)


def test_zero_weight_isolates_lora():
    wl = synth.tiny_layer(0)
    wl["W"] = np.zeros_like(wl.W)
    rng = np.random.default_rng(3)
    wl["x"] = synth.bf16_bits(rng.standard_normal((64, 256)).astype(np.float32))
    wl["dy"] = synth.bf16_bits(rng.standard_normal((64, 256)).astype(np.float32))
    for M in (8, 64):  # GEMV and GEMM paths
        qw, ref = _layer(wl)
        assert not ref["What"].any()
        x, dy = bf16_dev(wl.x[:M]), bf16_dev(wl.dy[:M])
        A, B = bf16_dev(wl.A), bf16_dev(wl.B)
        y = qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha)
        dx = qn.qlora_linear_bwd_dx(qw, dy, A, B, wl.r, wl.alpha)
        torch.cuda.synchronize()
        Z = np.zeros((256, 256))
        _check(f"lora-only y M={M}", to_np(y),
               linear.linear_forward(f64(wl.x[:M]), Z, f64(wl.A), f64(wl.B), wl.alpha, wl.r))
        _check(f"lora-only dx M={M}", to_np(dx),
               linear.linear_backward_input(f64(wl.dy[:M]), Z, f64(wl.A), f64(wl.B), wl.alpha, wl.r))


@pytest.mark.parametrize("M", [8, 64])
def test_b_zero_is_the_frozen_layer(M):
    wl = synth.tiny_layer(0)
    rng = np.random.default_rng(4)
    x = bf16_dev(synth.bf16_bits(rng.standard_normal((M, 256)).astype(np.float32)))
    dy = bf16_dev(synth.bf16_bits(rng.standard_normal((M, 256)).astype(np.float32)))
    qw, _ = _layer(wl)
    A = bf16_dev(wl.A)
    B0 = torch.zeros((256, wl.r), dtype=torch.bfloat16, device=x.device)
    y_lora = qn.qlora_linear_fwd(qw, x, A, B0, wl.r, wl.alpha)
    y_frozen = qn.qlora_linear_fwd(qw, x, None, None, 0, wl.alpha)
    dx_lora = qn.qlora_linear_bwd_dx(qw, dy, A, B0, wl.r, wl.alpha)
    dx_frozen = qn.qlora_linear_bwd_dx(qw, dy, None, None, 0, wl.alpha)
    dA, dB = qn.lora_grads(x, dy, A, B0, wl.r, wl.alpha)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits16(y_lora), to_bits16(y_frozen))
    assert np.array_equal(to_bits16(dx_lora), to_bits16(dx_frozen))
    assert not dA.any().item()
    assert dB.abs().sum().item() > 0


def test_frozen_layer_matches_oracle():
    wl = synth.tiny_layer(0)
    qw, ref = _layer(wl)
    for M in (16, 48):
        rng = np.random.default_rng(M)
        xb = synth.bf16_bits(rng.standard_normal((M, 256)).astype(np.float32))
        y = qn.qlora_linear_fwd(qw, bf16_dev(xb), None, None, 0, 1.0)
        torch.cuda.synchronize()
        _check(f"frozen y M={M}", to_np(y), f64(xb) @ ref["What"].astype(np.float64).T)


def test_empty_batch_is_a_no_op():
    wl = synth.tiny_layer(0)
    qw, _ = _layer(wl)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw, x, bf16_dev(wl.A), bf16_dev(wl.B), wl.r, wl.alpha)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


@pytest.mark.parametrize("N,K", [(192, 128), (320, 192)])
@pytest.mark.parametrize("M", [40, 300])
def test_ragged_output_columns(N, K, M):
    """Output widths that end in half a 128-column tile, and y at an element
    offset of 1 (rows not 8-byte aligned: element stores) or 4 (8-byte but not
    16-byte aligned: 8-byte stores from registers instead of the staged
    16-byte rows): every store path writes the same values."""
    wl = synth.train_linear(N, K, M=M, seed=N + M, r=8, alpha=16.0)
    run_layer_checks(wl, M=M)
    qw, _ = quantized_layer(wl)
    x, A, B = bf16_dev(wl.x), bf16_dev(wl.A), bf16_dev(wl.B)
    y = qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha)
    for off in (1, 4):
        buf = torch.zeros(M * N + off, dtype=torch.bfloat16, device=x.device)
        y_off = qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha, y=buf[off:].view(M, N))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits16(y_off), to_bits16(y)), f"offset {off}"
        assert not buf[:off].any().item()


@pytest.mark.parametrize("M", [8, 200])
def test_grads_recompute_matches_saved(M):
    """lora_grads without u and t recomputes them with the launches the
    forward and backward use for u_out and t_out: dA (through t) is the same
    bit for bit at any M, dB (through u) for token batches (M > 16)."""
    wl = synth.tiny_layer(0)
    rng = np.random.default_rng(500 + M)
    x = bf16_dev(synth.bf16_bits(rng.standard_normal((M, 256)).astype(np.float32)))
    dy = bf16_dev(synth.bf16_bits(rng.standard_normal((M, 256)).astype(np.float32)))
    qw, _ = quantized_layer(wl)
    A, B = bf16_dev(wl.A), bf16_dev(wl.B)
    u = torch.empty((M, wl.r), dtype=torch.bfloat16, device=x.device)
    t = torch.empty((M, wl.r), dtype=torch.bfloat16, device=x.device)
    qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha, u_out=u)
    qn.qlora_linear_bwd_dx(qw, dy, A, B, wl.r, wl.alpha, t_out=t)
    dA_s, dB_s = qn.lora_grads(x, dy, A, B, wl.r, wl.alpha, u=u, t=t)
    dA_r, dB_r = qn.lora_grads(x, dy, A, B, wl.r, wl.alpha)
    torch.cuda.synchronize()
    assert torch.equal(dA_s, dA_r)
    if M > 16:
        assert torch.equal(dB_s, dB_r)


@functools.lru_cache(maxsize=3)
def _decode_weight(N, K):
    """Device-quantised W (with and without double quantisation) and the
    oracle's fp32 dequantised weights, shared by the cases of one shape."""
    wl = synth.decode_layer(16, N, K, seed=2, r=64, alpha=16.0)
    w32 = synth.bf16_to_f32(wl.W)
    packed, absmax = nf4.quantize_nf4(w32)
    q8, c2 = nf4.double_quantize(absmax)
    What = {True: nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w32.size).reshape(N, K),
            False: nf4.dequantize(packed, absmax, w32.size).reshape(N, K)}
    wdev = bf16_dev(wl.W).reshape(N, K)
    qw = {True: qn.quantize_weight(wdev, True), False: qn.quantize_weight(wdev, False)}
    return wl, qw, What


@pytest.mark.parametrize("dq", [True, False], ids=["dq", "absmax"])
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("shape", [(8192, 22016), (22016, 8192), (8256, 4160)],
                         ids=["65b-down", "65b-gate", "uneven"])
def test_decode_gemv_long_rows(shape, M, dq):
    """Decode shapes whose rows take several passes of the GEMV's waves (the
    65B down and gate/up projections) and an uneven one (8256 x 4160: 65
    blocks per row, so a pass ends on a single block and some wave slices
    are empty), r = 64 so that M r exceeds the workgroup's thread count at
    M = 16; y and u_out against the oracle, with and without double
    quantisation of the block constants."""
    N, K = shape
    wl, qw, What = _decode_weight(N, K)
    x = wl.x[:M]
    u = torch.empty((M, wl.r), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw[dq], bf16_dev(x), bf16_dev(wl.A), bf16_dev(wl.B), wl.r, wl.alpha,
                            u_out=u)
    torch.cuda.synchronize()
    want = linear.linear_forward(f64(x), What[dq].astype(np.float64), f64(wl.A), f64(wl.B),
                                 wl.alpha, wl.r)
    _check(f"y {shape} M={M} dq={dq}", to_np(y), want)
    _check(f"u {shape} M={M}", to_np(u), linear.lora_down(f64(x), f64(wl.A)))


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("shape", [(8192, 22016), (22016, 8192), (8256, 4160)],
                         ids=["65b-down", "65b-gate", "uneven"])
def test_decode_gemv_long_rows_rank16(shape, M):
    """The long-row and uneven decode shapes at r = 16, alpha = 32 (the
    decode rank of the bench; M r then stays within the thread count, the
    other branch of the epilogue's u sum): y and u_out against the oracle,
    with the first 16 ranks of the shape's adapter."""
    N, K = shape
    wl, qw, What = _decode_weight(N, K)
    r, alpha = 16, 32.0
    x = wl.x[:M]
    A = np.ascontiguousarray(wl.A[:r])
    B = np.ascontiguousarray(wl.B[:, :r])
    u = torch.empty((M, r), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw[True], bf16_dev(x), bf16_dev(A), bf16_dev(B), r, alpha, u_out=u)
    torch.cuda.synchronize()
    want = linear.linear_forward(f64(x), What[True].astype(np.float64), f64(A), f64(B), alpha, r)
    _check(f"y {shape} r=16 M={M}", to_np(y), want)
    _check(f"u {shape} r=16 M={M}", to_np(u), linear.lora_down(f64(x), f64(A)))
