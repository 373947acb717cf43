"""Whole decoder layers at Llama-7B and 65B shapes (GPU).

Every projection is quantised on the device (NF4 + double quantisation of
the block constants) and compared bit for bit with the oracle's
quantisation of the same bf16 weight; then the QLoRA linear of that
projection runs forward, backward to the input and (7B) the LoRA gradients,
compared with the fp64 oracle to relative Frobenius error <= 1e-2 on sampled
token rows (a row of y or dx depends only on the same row of x or dy) and
in full for dA and dB.

Shapes: 7B ([kwkr] title and §1) and 65B ([rkmt] §1, §2.2.2) models; LoRA
on all seven linear projections of a block (q, k, v, o, gate, up, down: the
target-module list of [tgd]'s LoRA configuration); r = 64 with alpha = 16,
the setting [fg8] §8 reports.  Weights bf16 N(0, 0.02) (7B) and
N(0, 0.015) (65B).
"""

import numpy as np
import pytest

from tests.gpu_helpers import assert_quantized_equal, quantized_layer, run_layer_checks, synth

pytestmark = pytest.mark.gpu

R, ALPHA = 64, 16.0


def _rows(M, n, seed):
    return np.sort(np.random.default_rng(seed).choice(M, n, replace=False))


@pytest.mark.parametrize("idx", range(7), ids=[t[0] for t in synth.LLAMA7B_TARGETS])
def test_llama7b_layer_projection(idx):
    wl = synth.decoder_layer_linear(synth.LLAMA7B_TARGETS, idx, M=2048, r=R, alpha=ALPHA,
                                    std=0.02, seed=4)
    print(wl.name, flush=True)
    qw, ref = quantized_layer(wl)
    assert_quantized_equal(qw, ref)
    run_layer_checks(wl, rows=_rows(2048, 128, idx), qw=qw, ref=ref)


@pytest.mark.parametrize("idx", range(7), ids=[t[0] for t in synth.LLAMA65B_TARGETS])
def test_llama65b_layer_projection(idx):
    wl = synth.decoder_layer_linear(synth.LLAMA65B_TARGETS, idx, M=4096, r=R, alpha=ALPHA,
                                    std=0.015, seed=5)
    print(wl.name, flush=True)
    qw, ref = quantized_layer(wl)
    assert_quantized_equal(qw, ref)
    run_layer_checks(wl, rows=_rows(4096, 64, 100 + idx), grads=False, qw=qw, ref=ref)


@pytest.mark.parametrize("idx", [0, 4, 6], ids=["q", "gate", "down"])
def test_llama7b_projection_rank128(idx):
    """r = 128 with alpha = 32 ([fg8] §8): the fused GEMMs' LoRA contraction
    in two 64-deep passes, the 128-column LoRA projections and gradients."""
    wl = synth.decoder_layer_linear(synth.LLAMA7B_TARGETS, idx, M=2048, r=128, alpha=32.0,
                                    std=0.02, seed=4)
    print(wl.name, flush=True)
    qw, ref = quantized_layer(wl)
    run_layer_checks(wl, rows=_rows(2048, 128, 50 + idx), qw=qw, ref=ref)
