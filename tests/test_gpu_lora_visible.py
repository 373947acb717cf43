"""The LoRA terms on their own, at the ranks the layers use (GPU).

At the layer settings (r = 64, alpha = 16, A and B ~ N(0, 0.01)) the
adapter's share of y and dx is about 1%, below what a 1e-2 relative
Frobenius check of the whole output can see.  With W = 0 every code is the
exact zero (code 7) and the block constants are 0, so the layer is the
adapter alone ([rkmt] §2.1: the frozen weight plus the low-rank product
B A; [rkmt] §3.3: scaled by alpha / r):
  y  = s (x A^T) B^T,   dx = s (dy B) A,   dA = s (dy B)^T x,  dB = s dy^T (x A^T)
and each output is compared with the fp64 oracle on its own.  This covers
the decode GEMV's LoRA epilogue (M <= 16, including M r above the
workgroup's thread count), the fused GEMM's LoRA contraction in both
directions past the first 16 ranks (r = 32, 64, 100, 128) and the LoRA
gradients at those ranks.  r = 128 with alpha = 32 is the setting [fg8] §8
reports.  The smallest ranks (r = 1, 3: one MFMA column tile, 15 or 13 of
its 16 columns padding) and r = 17 (one rank past the GEMM's 16-wide early
LoRA tile, so the late contraction with a 16-deep step that is almost all
padding) check the rank edges.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import bf16_dev, check, f64, linear, synth, to_np

pytestmark = pytest.mark.gpu

N, K = 1088, 2112    # 8.5 column tiles of 128 (ragged), 33 quantisation blocks per row
RANKS = [(1, 2.0), (3, 6.0), (17, 16.0), (32, 16.0), (64, 16.0), (100, 16.0), (128, 32.0)]


def _zero_weight():
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda:0")
    return qn.quantize_weight(w)


def _inputs(M, r, seed):
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    dy = synth.bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    A = synth.bf16_bits((rng.standard_normal((r, K)) * 0.01).astype(np.float32))
    B = synth.bf16_bits((rng.standard_normal((N, r)) * 0.01).astype(np.float32))
    return x, dy, A, B


@pytest.mark.parametrize("r,alpha", RANKS, ids=[f"r{r}" for r, _ in RANKS])
@pytest.mark.parametrize("M", [1, 16, 64, 2048])
def test_lora_only_forward(r, alpha, M):
    qw = _zero_weight()
    x, _, A, B = _inputs(M, r, 7000 + 10 * r + M)
    u = torch.empty((M, r), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw, bf16_dev(x), bf16_dev(A), bf16_dev(B), r, alpha, u_out=u)
    torch.cuda.synchronize()
    Z = np.zeros((N, K))
    check(f"lora-only y r={r} M={M}", to_np(y),
          linear.linear_forward(f64(x), Z, f64(A), f64(B), alpha, r))
    check(f"u r={r} M={M}", to_np(u), linear.lora_down(f64(x), f64(A)))


@pytest.mark.parametrize("r,alpha", RANKS, ids=[f"r{r}" for r, _ in RANKS])
@pytest.mark.parametrize("M", [16, 64, 2048])
def test_lora_only_backward_and_grads(r, alpha, M):
    qw = _zero_weight()
    x, dy, A, B = _inputs(M, r, 8000 + 10 * r + M)
    t = torch.empty((M, r), dtype=torch.bfloat16, device="cuda:0")
    dxt, dyt, At, Bt = bf16_dev(x), bf16_dev(dy), bf16_dev(A), bf16_dev(B)
    dx = qn.qlora_linear_bwd_dx(qw, dyt, At, Bt, r, alpha, t_out=t)
    dA, dB = qn.lora_grads(dxt, dyt, At, Bt, r, alpha)
    torch.cuda.synchronize()
    Z = np.zeros((N, K))
    check(f"lora-only dx r={r} M={M}", to_np(dx),
          linear.linear_backward_input(f64(dy), Z, f64(A), f64(B), alpha, r))
    check(f"t r={r} M={M}", to_np(t), linear.lora_up_input(f64(dy), f64(B)))
    rA, rB = linear.lora_grads(f64(x), f64(dy), f64(A), f64(B), alpha, r)
    check(f"dA r={r} M={M}", to_np(dA), rA)
    # dB [N, r] is checked per rank, over its N outputs: a row of dB holds
    # only r values, and at r = 1 the largest-element-over-row-norm bound
    # would become one element's relative error, which a cancelling sum of
    # M products with the bf16 u exceeds at M = 16
    check(f"dB r={r} M={M} (per rank)", to_np(dB).T, rB.T)


@pytest.mark.parametrize("M", [1, 64])
def test_null_adapter_pointers_are_the_frozen_layer(M):
    """A == B == NULL with r > 0 runs the frozen layer: bit for bit the r = 0
    result, forward and backward."""
    wl = synth.train_linear(256, 320, M=M, seed=77, r=16, alpha=32.0)
    qw = qn.quantize_weight(bf16_dev(wl.W).reshape(256, 320))
    x, dy = bf16_dev(wl.x), bf16_dev(wl.dy)
    y0 = qn.qlora_linear_fwd(qw, x, None, None, 0, 32.0)
    dx0 = qn.qlora_linear_bwd_dx(qw, dy, None, None, 0, 32.0)
    y1 = torch.empty_like(y0)
    dx1 = torch.empty_like(dx0)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    qn.qlora_linear_fwd(qw, x, None, None, 16, 32.0, y=y1, ws=ws)
    qn.qlora_linear_bwd_dx(qw, dy, None, None, 16, 32.0, dx=dx1, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(dx0, dx1)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("shape", [(11008, 4096), (8192, 22016), (4096, 4096)],
                         ids=["11008x4096", "8192x22016", "4096x4096"])
def test_lora_only_decode_rank16(shape, M):
    """W = 0 at decode shapes and r = 16, the decode rank of the bench: the
    LoRA-down launch's partial sums as the GEMV's epilogue adds them up
    (11008 x 4096 at M = 1 and 8192 x 22016 take several GEMV passes), and
    at 4096 x 4096, M = 1, u computed inside the GEMV launch from the x
    slices it stages."""
    n, k = shape
    r, alpha = 16, 32.0
    qw = qn.quantize_weight(torch.zeros((n, k), dtype=torch.bfloat16, device="cuda:0"))
    rng = np.random.default_rng(9100 + M + n // 64)
    x = synth.bf16_bits(rng.standard_normal((M, k), dtype=np.float32))
    A = synth.bf16_bits((rng.standard_normal((r, k)) * 0.01).astype(np.float32))
    B = synth.bf16_bits((rng.standard_normal((n, r)) * 0.01).astype(np.float32))
    u = torch.empty((M, r), dtype=torch.bfloat16, device="cuda:0")
    y = qn.qlora_linear_fwd(qw, bf16_dev(x), bf16_dev(A), bf16_dev(B), r, alpha, u_out=u)
    torch.cuda.synchronize()
    check(f"lora-only y {shape} r=16 M={M}", to_np(y),
          linear.linear_forward(f64(x), np.zeros((n, k)), f64(A), f64(B), alpha, r))
    check(f"u {shape} r=16 M={M}", to_np(u), linear.lora_down(f64(x), f64(A)))


GRAD_CASES = [(8, 16.0, 1), (16, 32.0, 200), (24, 16.0, 1000), (64, 16.0, 4095), (128, 32.0, 130),
              (32, 16.0, 0)]


@pytest.mark.parametrize("r,alpha,M", GRAD_CASES,
                         ids=[f"r{r}-M{M}" for r, _, M in GRAD_CASES])
def test_lora_grads_token_edges(r, alpha, M):
    """LoRA gradients where the token count ends inside a 64-token step and
    the steps do not divide evenly over a workgroup's waves (M = 1, 200,
    1000, 4095), ranks below the rank tile (r = 24 of 32), and no tokens
    (M = 0: both gradients are exactly zero).  With r % 8 == 0 and u, t
    16-byte aligned the column-tile launch runs; u and t passed one element
    off 16-byte alignment take the token-chunk launches and its reduction,
    and both must match the fp64 oracle."""
    x, dy, A, B = _inputs(M, r, 9000 + 10 * r + M)
    dxt, dyt, At, Bt = bf16_dev(x), bf16_dev(dy), bf16_dev(A), bf16_dev(B)
    rA, rB = linear.lora_grads(f64(x), f64(dy), f64(A), f64(B), alpha, r)
    u_ref = synth.bf16_bits(linear.lora_down(f64(x), f64(A)).astype(np.float32))
    t_ref = synth.bf16_bits(linear.lora_up_input(f64(dy), f64(B)).astype(np.float32))
    runs = {"own u, t": qn.lora_grads(dxt, dyt, At, Bt, r, alpha)}
    for off in (0, 1):
        ub = torch.zeros(M * r + off, dtype=torch.bfloat16, device="cuda:0")
        tb = torch.zeros(M * r + off, dtype=torch.bfloat16, device="cuda:0")
        u = ub[off:].view(M, r)
        t = tb[off:].view(M, r)
        u.copy_(bf16_dev(u_ref))
        t.copy_(bf16_dev(t_ref))
        runs[f"u, t at +{off}"] = qn.lora_grads(dxt, dyt, At, Bt, r, alpha, u=u, t=t)
    torch.cuda.synchronize()
    for name, (dA, dB) in runs.items():
        if M == 0:
            assert not torch.any(dA) and not torch.any(dB), name
            continue
        check(f"dA r={r} M={M} {name}", to_np(dA), rA)
        check(f"dB r={r} M={M} {name} (per rank)", to_np(dB).T, rB.T)


@pytest.mark.parametrize("NK,r,M", [((1024, 1024), 32, 300), ((512, 1536), 64, 2048)],
                         ids=["1024x1024-r32", "512x1536-r64"])
def test_lora_grads_paired_column_tiles(NK, r, M):
    """32-column gradient tiles with both tile counts multiples of 16, where
    each group of 16 workgroups takes its tiles as adjacent pairs (one XCD
    per pair): every column of dA and dB is written once, with its own sum."""
    n, k = NK
    rng = np.random.default_rng(9500 + r + M)
    x = synth.bf16_bits(rng.standard_normal((M, k), dtype=np.float32))
    dy = synth.bf16_bits(rng.standard_normal((M, n), dtype=np.float32))
    A = synth.bf16_bits((rng.standard_normal((r, k)) * 0.01).astype(np.float32))
    B = synth.bf16_bits((rng.standard_normal((n, r)) * 0.01).astype(np.float32))
    dA, dB = qn.lora_grads(bf16_dev(x), bf16_dev(dy), bf16_dev(A), bf16_dev(B), r, 16.0)
    torch.cuda.synchronize()
    rA, rB = linear.lora_grads(f64(x), f64(dy), f64(A), f64(B), 16.0, r)
    check(f"dA paired tiles {n}x{k} r={r} M={M}", to_np(dA), rA)
    check(f"dB paired tiles {n}x{k} r={r} M={M} (per rank)", to_np(dB).T, rB.T)
