"""Pins for the oracle's QLoRA linear layer (CPU only).

The oracle uses numpy matrix products; these tests tie it to the definition
by brute force on tiny shapes (pure-Python sums), to exact special cases
(B = 0, W = 0, unit-vector inputs), and tie backward and gradients to the
forward map by exact directional derivatives (the layer is linear in x, A
and B separately, so a finite difference in fp64 is exact up to rounding).
Non-square shapes everywhere so a transposed operand cannot pass.
"""

import numpy as np
import pytest

from oracle import linear, nf4


def _case(M=3, N=5, K=7, r=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.1
    A = rng.standard_normal((r, K)) * 0.3
    B = rng.standard_normal((N, r)) * 0.3
    dy = rng.standard_normal((M, N))
    return x, W, A, B, dy


def _brute_forward(x, W, A, B, alpha, r):
    M, K = x.shape
    N = W.shape[0]
    s = alpha / r
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += x[m][k] * W[n][k]
            lora = 0.0
            for j in range(r):
                u = 0.0
                for k in range(K):
                    u += A[j][k] * x[m][k]
                lora += B[n][j] * u
            y[m][n] = acc + s * lora
    return np.array(y)


def test_forward_matches_brute_force():
    x, W, A, B, _ = _case()
    y = linear.linear_forward(x, W, A, B, alpha=3.0, r=2)
    assert y.shape == (3, 5)
    assert np.allclose(y, _brute_forward(x, W, A, B, 3.0, 2), rtol=1e-13, atol=1e-13)


def test_backward_input_matches_brute_force():
    x, W, A, B, dy = _case(seed=1)
    dx = linear.linear_backward_input(dy, W, A, B, alpha=3.0, r=2)
    M, K = x.shape
    want = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            v = 0.0
            for n in range(W.shape[0]):
                v += dy[m][n] * W[n][k]
                for j in range(2):
                    v += 1.5 * dy[m][n] * B[n][j] * A[j][k]
            want[m][k] = v
    assert np.allclose(dx, want, rtol=1e-13, atol=1e-13)


def _inner(a, b):
    return float(np.sum(a * b))


@pytest.mark.parametrize("seed", [2, 3])
def test_adjoints_and_gradients_are_exact_derivatives(seed):
    x, W, A, B, dy = _case(M=4, N=6, K=9, r=3, seed=seed)
    alpha = 6.0
    rng = np.random.default_rng(100 + seed)
    f = lambda x_, A_, B_: _inner(dy, linear.linear_forward(x_, W, A_, B_, alpha, 3))
    base = f(x, A, B)
    dx = linear.linear_backward_input(dy, W, A, B, alpha, 3)
    dA, dB = linear.lora_grads(x, dy, A, B, alpha, 3)
    for target, grad in (("x", dx), ("A", dA), ("B", dB)):
        V = rng.standard_normal(grad.shape)
        if target == "x":
            d = f(x + V, A, B) - base
        elif target == "A":
            d = f(x, A + V, B) - base
        else:
            d = f(x, A, B + V) - base
        assert abs(d - _inner(grad, V)) < 1e-10 * (1 + abs(d))


def test_b_zero_is_the_frozen_layer():
    x, W, A, B, dy = _case(seed=4)
    B0 = np.zeros_like(B)
    y = linear.linear_forward(x, W, A, B0, 16.0, 2)
    assert np.array_equal(y, x @ W.T)
    dA, dB = linear.lora_grads(x, dy, A, B0, 16.0, 2)
    assert np.all(dA == 0)
    assert np.any(dB != 0)
    assert np.array_equal(linear.linear_backward_input(dy, W, A, B0, 16.0, 2), dy @ W)


def test_zero_weight_isolates_the_lora_term():
    # W = 0 quantises to code 7 everywhere, which dequantises to exact zeros.
    packed, absmax = nf4.quantize_nf4(np.zeros(5 * 64, np.float32))
    W = nf4.dequantize(packed, absmax, 5 * 64).reshape(5, 64)
    assert np.all(W == 0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64))
    A = rng.standard_normal((2, 64))
    B = rng.standard_normal((5, 2))
    y = linear.linear_forward(x, W, A, B, 4.0, 2)
    assert np.allclose(y, _brute_forward(x, np.zeros((5, 64)), A, B, 4.0, 2), rtol=1e-13)


def test_unit_vector_inputs_read_columns():
    # x = e_k picks column k of W plus s * B A[:, k].
    x, W, A, B, _ = _case(M=7, N=5, K=7, r=2, seed=6)
    y = linear.linear_forward(np.eye(7), W, A, B, 5.0, 2)
    for k in range(7):
        want = W[:, k] + 2.5 * (B @ A[:, k])
        assert np.allclose(y[k], want, rtol=1e-14, atol=1e-15)


def test_scale_is_alpha_over_r():
    x, W, A, B, _ = _case(seed=7)
    y1 = linear.linear_forward(x, W, A, B, 2.0, 2)
    y2 = linear.linear_forward(x, W, A, B, 4.0, 2)
    base = linear.linear_forward(x, W, A, np.zeros_like(B), 2.0, 2)
    assert np.allclose(y2 - base, 2 * (y1 - base), rtol=1e-12)
    # alpha = r gives unit scale: the bypass is exactly B A x
    y3 = linear.linear_forward(x, W, A, B, 2.0, 2)
    assert np.allclose(y3 - base, x @ (B @ A).T, rtol=1e-12)


def test_rank_zero_is_frozen():
    x, W, _, _, dy = _case(seed=8)
    y = linear.linear_forward(x, W, None, None, 16.0, 0)
    assert np.array_equal(y, x @ W.T)


def test_cross_check_with_torch_fp64_on_a_dequantised_weight():
    """The oracle's forward, backward to the input and LoRA gradients equal
    torch's CPU fp64 autograd of the same layer, y = x W^T + s (x A^T) B^T,
    on an NF4-dequantised W (an independent library implementation of the
    products and of the chain rule: dx, dA and dB come from torch's
    backward, not from the oracle's formulas)."""
    import torch

    rng = np.random.default_rng(31)
    M, N, K, r, alpha = 9, 192, 128, 4, 8.0
    w = (rng.standard_normal(N * K) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize_nf4(w)
    q8, c2 = nf4.double_quantize(absmax)
    What = nf4.dequantize(packed, nf4.dequant_scales(q8, c2), w.size).reshape(N, K)
    x = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dy = rng.standard_normal((M, N))
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    tB = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(What.astype(np.float64))
    ty = torch.nn.functional.linear(tx, tW) + (alpha / r) * torch.nn.functional.linear(
        torch.nn.functional.linear(tx, tA), tB)
    ty.backward(torch.tensor(dy))
    y = linear.linear_forward(x, What, A, B, alpha, r)
    dx = linear.linear_backward_input(dy, What, A, B, alpha, r)
    dA, dB = linear.lora_grads(x, dy, A, B, alpha, r)
    for got, want in ((y, ty.detach()), (dx, tx.grad), (dA, tA.grad), (dB, tB.grad)):
        assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
