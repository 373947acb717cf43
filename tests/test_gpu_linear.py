"""Parity of the QLoRA linear layer (forward, backward to the input, LoRA
gradients) with the fp64 CPU oracle (GPU).

Bar: relative Frobenius error <= 1e-2 per output (bf16 operands, fp32
accumulation).  The oracle multiplies the exact fp32 dequantised weight in
fp64; the HIP path rounds it to bf16 for the MFMA, so the expected error is
the bf16 rounding of weights, activations and outputs (~1e-3).
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import (bf16_dev, f32_dev, f64, linear, oracle_quant, rel_frob, synth,
                               to_bits16, to_np, weight_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _layer(wl, double_quant=True):
    qw = qn.quantize_weight(weight_dev(wl.W, wl.W_dtype).reshape(wl.N, wl.K), double_quant)
    ref = oracle_quant(wl.W, wl.W_dtype, double_quant)
    return qw, ref


def _check(name, got, ref, tol=TOL):
    e = rel_frob(got, ref)
    print(f"{name}: rel_frob={e:.3e}")
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol}"


def _run_all(wl, M=None, rows=None, double_quant=True):
    M = wl.M if M is None else M
    qw, ref = _layer(wl, double_quant)
    x_bits, dy_bits = wl.x[:M], wl.dy[:M]
    x, A, B, dy = bf16_dev(x_bits), bf16_dev(wl.A), bf16_dev(wl.B), bf16_dev(dy_bits)
    u_out = torch.empty((M, wl.r), dtype=torch.bfloat16, device=x.device)
    t_out = torch.empty((M, wl.r), dtype=torch.bfloat16, device=x.device)
    y = qn.qlora_linear_fwd(qw, x, A, B, wl.r, wl.alpha, u_out=u_out)
    dx = qn.qlora_linear_bwd_dx(qw, dy, A, B, wl.r, wl.alpha, t_out=t_out)
    dA, dB = qn.lora_grads(x, dy, A, B, wl.r, wl.alpha)
    dA2, dB2 = qn.lora_grads(x, dy, A, B, wl.r, wl.alpha, u=u_out, t=t_out)
    torch.cuda.synchronize()
    xf, dyf, Af, Bf = f64(x_bits), f64(dy_bits), f64(wl.A), f64(wl.B)
    sel = np.arange(M) if rows is None else rows
    What = ref["What"].astype(np.float64)
    _check("y", to_np(y)[sel], linear.linear_forward(xf[sel], What, Af, Bf, wl.alpha, wl.r))
    _check("dx", to_np(dx)[sel], linear.linear_backward_input(dyf[sel], What, Af, Bf, wl.alpha, wl.r))
    rA, rB = linear.lora_grads(xf, dyf, Af, Bf, wl.alpha, wl.r)
    _check("dA", to_np(dA), rA)
    _check("dB", to_np(dB), rB)
    _check("dA(saved u,t)", to_np(dA2), rA)
    _check("dB(saved u,t)", to_np(dB2), rB)
    _check("u", to_np(u_out)[sel], linear.lora_down(xf[sel], Af))
    _check("t", to_np(t_out)[sel], linear.lora_up_input(dyf[sel], Bf))


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
