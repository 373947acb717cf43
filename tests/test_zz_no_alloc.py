"""The allocation-free forward against qlora_linear_fwd (GPU).

qlora_linear_fwd_noalloc runs the forward's own kernels on the library's
per-GPU scratch array instead of a caller workspace, so y and u_out must
equal qlora_linear_fwd's bit for bit.  Each case makes two calls in a row on
the same array, the second with a smaller input, so the second reads an
array that still holds the first call's partial sums: nothing in it may be
taken to start at zero.  Token-batch (fused GEMM) and decode (GEMV) paths
both use the array for the LoRA-down partial sums.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _layer(N, K, r, seed):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    A = torch.from_numpy(synth.bf16_bits((rng.standard_normal((r, K)) * 0.01).astype(np.float32))
                         .view(np.int16)).view(torch.bfloat16).to(DEV)
    B = torch.from_numpy(synth.bf16_bits((rng.standard_normal((N, r)) * 0.01).astype(np.float32))
                         .view(np.int16)).view(torch.bfloat16).to(DEV)
    return qn.quantize_weight(W), A, B


def _x(M, K, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(synth.bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
                            .view(np.int16)).view(torch.bfloat16).to(DEV)


def _both(qw, x, A, B, r, alpha):
    M = x.shape[0]
    y_ref = torch.empty((M, qw.N), dtype=torch.bfloat16, device=DEV)
    u_ref = torch.empty((M, r), dtype=torch.bfloat16, device=DEV)
    qn.qlora_linear_fwd(qw, x, A, B, r, alpha, y=y_ref, u_out=u_ref)
    y = torch.full((M, qw.N), float("nan"), dtype=torch.bfloat16, device=DEV)
    u = torch.full((M, r), float("nan"), dtype=torch.bfloat16, device=DEV)
    qn.qlora_linear_fwd_noalloc(qw, x, A, B, r, alpha, y, u_out=u)
    torch.cuda.synchronize()
    return y_ref, u_ref, y, u


# (N, K, r, alpha, first M, second M): token batches on the fused GEMM, then
# decode calls on the GEMV, each followed by a smaller call
CASES = [
    (1088, 2112, 64, 16.0, 2048, 320),
    (4096, 4096, 64, 16.0, 4096, 16),
    (4096, 11008, 16, 32.0, 16, 1),
    (1088, 2112, 128, 32.0, 64, 4),
    (1088, 2112, 16, 32.0, 16, 1),  # the second call computes u inside the GEMV launch
]


@pytest.mark.parametrize("N,K,r,alpha,M1,M2", CASES)
def test_noalloc_forward_matches_the_workspace_forward(N, K, r, alpha, M1, M2):
    qw, A, B = _layer(N, K, r, seed=N + K + r)
    for call, M in enumerate((M1, M2)):
        x = _x(M, K, seed=100 * call + M)
        y_ref, u_ref, y, u = _both(qw, x, A, B, r, alpha)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (call, M)
        assert torch.equal(u.view(torch.int16), u_ref.view(torch.int16)), (call, M)


def test_noalloc_frozen_layer_and_repeated_calls():
    """r = 0 needs no scratch; repeated calls of one size give the same bits."""
    qw, A, B = _layer(1088, 2112, 32, seed=7)
    x = _x(48, 2112, seed=8)
    y0 = torch.empty((48, 1088), dtype=torch.bfloat16, device=DEV)
    qn.qlora_linear_fwd(qw, x, None, None, 0, 1.0, y=y0)
    y1 = torch.empty_like(y0)
    qn.qlora_linear_fwd_noalloc(qw, x, None, None, 0, 1.0, y1)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    first = None
    for _ in range(3):
        y = torch.empty_like(y0)
        qn.qlora_linear_fwd_noalloc(qw, x, A, B, 32, 16.0, y)
        torch.cuda.synchronize()
        if first is None:
            first = y
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))


def test_noalloc_rejects_sizes_beyond_the_array():
    qw, A, B = _layer(1088, 2112, 128, seed=9)
    M = 8192  # forward workspace of M r = 2^20 rows x ranks: 66 MiB > 64 MiB
    x = torch.zeros((M, 2112), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((M, 1088), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qn.QnError) as e:
        qn.qlora_linear_fwd_noalloc(qw, x, A, B, 128, 32.0, y)
    assert e.value.status == qn.QN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not y.any()
