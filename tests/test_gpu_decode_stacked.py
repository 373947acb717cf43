"""Projections that read the same input, run as one call on stacked weights
(GPU).

q, k and v of an attention block read the same x, and so do gate and up of
the MLP ([rkmt] §2.1 puts LoRA on the attention and MLP projections, and the
LoRA configuration of its §3.3 targets all seven).  Their
weights stacked by rows form one [n N, K] weight whose 64-blocks and
256-block double-quantisation groups are those of the separate weights
(N K / 64 a multiple of 256), so quantising the stack gives the separate
codes and constants byte for byte.  The adapters stack as one of rank n r:
A = [A_1; ...; A_n] and a block-diagonal B (B_j in rows j N .. and columns
j r ..), with alpha scaled by n so that alpha / r is unchanged; then
x A^T B^T is the separate LoRA terms side by side, and one
qlora_linear_fwd call computes all n projections.  Checked against the
oracle's separate layers and against the separate library calls.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import bf16_dev, check, f64, linear, oracle_quant, synth, to_np

pytestmark = pytest.mark.gpu

N, K, R, ALPHA = 1024, 2048, 16, 32.0


@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_stacked_projections(n, M):
    rng = np.random.default_rng(500 + 10 * n + M)
    Ws = [synth.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
          for _ in range(n)]
    As = [synth.bf16_bits((rng.standard_normal((R, K)) * 0.05).astype(np.float32))
          for _ in range(n)]
    Bs = [synth.bf16_bits((rng.standard_normal((N, R)) * 0.05).astype(np.float32))
          for _ in range(n)]
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))

    sep = [qn.quantize_weight(bf16_dev(W).reshape(N, K)) for W in Ws]
    stk = qn.quantize_weight(bf16_dev(np.concatenate(Ws)).reshape(n * N, K))
    torch.cuda.synchronize()
    for attr in ("packed", "qscale", "gscale"):
        want = torch.cat([getattr(q, attr).reshape(-1) for q in sep])
        assert torch.equal(getattr(stk, attr).reshape(-1), want), attr

    B_bd = np.zeros((n * N, n * R), dtype=np.uint16)  # bf16 +0.0
    for j, B in enumerate(Bs):
        B_bd[j * N:(j + 1) * N, j * R:(j + 1) * R] = B
    xd = bf16_dev(x)
    y_stk = qn.qlora_linear_fwd(stk, xd, bf16_dev(np.concatenate(As)), bf16_dev(B_bd), n * R,
                                n * ALPHA)
    y_sep = [qn.qlora_linear_fwd(q, xd, bf16_dev(A), bf16_dev(B), R, ALPHA)
             for q, A, B in zip(sep, As, Bs)]
    torch.cuda.synchronize()
    got = to_np(y_stk)
    for j in range(n):
        What = oracle_quant(Ws[j], "bf16")["What"]
        want = linear.linear_forward(f64(x), What, f64(As[j]), f64(Bs[j]), ALPHA, R)
        part = got[:, j * N:(j + 1) * N]
        check(f"stacked y[{j}] n={n} M={M}", part, want)
        check(f"stacked y[{j}] against the separate call n={n} M={M}", part, to_np(y_sep[j]))
