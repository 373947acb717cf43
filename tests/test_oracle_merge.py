"""Pins of the oracle's LoRA merge and of its fp64 -> bf16 rounding (CPU).

The merged weight must reproduce the LoRA forward ([rkmt] §2.1: folding the
adapter into the weight leaves the output unchanged), reduce to the
dequantised weight when B = 0, and change exactly one entry for a rank-1
update with one-hot factors.
"""

import numpy as np

from bit_nf4_quantized_22_amd import synth
from oracle import linear, nf4


def _layer(seed=7, N=48, K=128, r=4):
    rng = np.random.default_rng(seed)
    w_hat = (rng.standard_normal((N, K)) * 0.02).astype(np.float32).astype(np.float64)
    A = rng.standard_normal((r, K)) * 0.01
    B = rng.standard_normal((N, r)) * 0.01
    return w_hat, A, B


def test_merged_weight_reproduces_lora_forward():
    w_hat, A, B = _layer()
    x = np.random.default_rng(8).standard_normal((5, w_hat.shape[1]))
    merged = linear.lora_merge(w_hat, A, B, 16.0, 4)
    y_merged = x @ merged.T
    y_lora = linear.linear_forward(x, w_hat, A, B, 16.0, 4)
    assert np.allclose(y_merged, y_lora, rtol=0, atol=1e-13)


def test_b_zero_merge_is_the_dequantised_weight():
    w_hat, A, B = _layer()
    merged = linear.lora_merge(w_hat, A, np.zeros_like(B), 16.0, 4)
    assert np.array_equal(merged, w_hat)
    assert np.array_equal(nf4.f64_to_bf16_bits(merged), nf4.f32_to_bf16_bits(w_hat.astype(np.float32)))


def test_rank_one_one_hot_changes_one_entry():
    w_hat, _, _ = _layer()
    N, K = w_hat.shape
    A = np.zeros((1, K)); A[0, 17] = 0.25
    B = np.zeros((N, 1)); B[5, 0] = -3.0
    merged = linear.lora_merge(w_hat, A, B, 2.0, 1)  # s = 2
    diff = merged - w_hat
    assert diff[5, 17] == 2.0 * -3.0 * 0.25
    diff[5, 17] = 0.0
    assert not np.any(diff)


def test_f64_to_bf16_matches_fp32_rounding_on_fp32_values():
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0, -2.5, 65504.0]]).astype(np.float32)
    assert np.array_equal(nf4.f64_to_bf16_bits(v.astype(np.float64)), nf4.f32_to_bf16_bits(v))


def test_f64_to_bf16_ties_and_sticky_bits():
    one = 1.0
    # halfway between 1 and 1 + 2^-7 rounds to the even 1.0; anything above goes up
    assert nf4.f64_to_bf16_bits(np.array([one + 2.0 ** -8]))[0] == 0x3F80
    assert nf4.f64_to_bf16_bits(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    # halfway between 1 + 2^-7 (odd) and 1 + 2^-6 rounds up to the even one
    assert nf4.f64_to_bf16_bits(np.array([one + 3 * 2.0 ** -8]))[0] == 0x3F82
    # a value just above an fp32 tie: rounding through fp32 first would lose the sticky bit
    x = one + 2.0 ** -8 + 2.0 ** -50
    assert nf4.f64_to_bf16_bits(np.array([x]))[0] == 0x3F81
    assert nf4.f32_to_bf16_bits(np.array([x], dtype=np.float32))[0] == 0x3F80


def test_merge_on_a_quantised_layer_rounds_like_the_direct_definition():
    wl = synth.tiny_layer(0)
    packed, absmax = nf4.quantize_nf4(wl.W)
    q8, c2 = nf4.double_quantize(absmax)
    w_hat = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), wl.W.size).reshape(wl.N, wl.K)
    A = synth.bf16_to_f32(wl.A).astype(np.float64)
    B = synth.bf16_to_f32(wl.B).astype(np.float64)
    merged = linear.lora_merge(w_hat, A, B, wl.alpha, wl.r)
    bits = nf4.f64_to_bf16_bits(merged)
    back = nf4.bf16_bits_to_f32(bits).astype(np.float64)
    # nearest bf16: within half a bf16 spacing of the fp64 value
    _, e = np.frexp(merged)
    assert np.all(np.abs(back - merged) <= np.ldexp(1.0, np.maximum(e - 9, -134)))
