"""Seeded synthetic inputs shared by the tests, the smoke run and the bench.

This module holds no arithmetic of the method: it only draws random numbers
(numpy PCG64, ``default_rng(seed)``) and rounds them to the storage types of
the inputs (fp32, or bf16 by round-to-nearest-even).  Both the HIP path and
the CPU oracle receive the same arrays from here.

Draw order inside one workload: W (one tensor per projection, in the order
listed), x, A, B, dy.  Weights are drawn in fp32 and, for bf16 workloads,
rounded to bf16; activations, gradients and LoRA matrices are bf16.
"""

import numpy as np

# Llama-7B and 65B-shaped projections: (name, N = out_features, K = in_features)
LLAMA7B_TARGETS = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
                   ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
                   ("down", 4096, 11008)]
LLAMA65B_TARGETS = [("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192),
                    ("o", 8192, 8192), ("gate", 22016, 8192), ("up", 22016, 8192),
                    ("down", 8192, 22016)]


def bf16_bits(x):
    """Round fp32 values to bf16 (RNE) and return the uint16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std):
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = rng.standard_normal(n, dtype=np.float32) * np.float32(std)
    return out


def _student_t(rng, shape, df, std):
    # Student-t(df) has variance df/(df-2); scale to the requested std.
    scale = std / np.sqrt(df / (df - 2.0))
    return (rng.standard_t(df, size=shape) * scale).astype(np.float32)


class Workload(dict):
    """A dict of named arrays plus scalar settings (attribute access too)."""

    __getattr__ = dict.__getitem__


def tiny_layer(seed=0):
    """W 256x256 fp32 N(0, 0.02); x 16x256 bf16 N(0,1); r=8, alpha=16;
    A, B N(0, 0.01); dy 16x256 bf16 N(0, 1)."""
    rng = np.random.default_rng(seed)
    W = _normal(rng, (256, 256), 0.02)
    x = bf16_bits(_normal(rng, (16, 256), 1.0))
    A = bf16_bits(_normal(rng, (8, 256), 0.01))
    B = bf16_bits(_normal(rng, (256, 8), 0.01))
    dy = bf16_bits(_normal(rng, (16, 256), 1.0))
    return Workload(name="tiny 256x256 fp32, M=16, r=8", W=W, W_dtype="f32", x=x,
                    A=A, B=B, dy=dy, M=16, N=256, K=256, r=8, alpha=16.0)


def decode_layer(M, N=4096, K=4096, seed=2, r=16, alpha=32.0, std=0.02):
    """Decode GEMV: W NxK bf16 N(0, std); x Mx K bf16 N(0,1); r=16, alpha=32;
    A, B N(0, 0.01) (the LoRA distribution of the tiny layer, a reading)."""
    rng = np.random.default_rng(seed)
    W = bf16_bits(_normal(rng, (N, K), std))
    x = bf16_bits(_normal(rng, (M, K), 1.0))
    A = bf16_bits(_normal(rng, (r, K), 0.01))
    B = bf16_bits(_normal(rng, (N, r), 0.01))
    return Workload(name=f"decode W {N}x{K} bf16, M={M}, r={r}", W=W, W_dtype="bf16",
                    x=x, A=A, B=B, dy=None, M=M, N=N, K=K, r=r, alpha=alpha)


def train_linear(N, K, M=2048, seed=3, r=16, alpha=32.0, heavy_tail=True, std=0.02):
    """Training-step linear: W NxK Student-t(5) scaled to std 0.02 (absmax
    outliers) or normal, bf16; x MxK and dy MxN bf16 N(0,1); A, B N(0, 0.01)."""
    rng = np.random.default_rng(seed)
    if heavy_tail:
        W = bf16_bits(_student_t(rng, (N, K), 5, std))
    else:
        W = bf16_bits(_normal(rng, (N, K), std))
    x = bf16_bits(_normal(rng, (M, K), 1.0))
    A = bf16_bits(_normal(rng, (r, K), 0.01))
    B = bf16_bits(_normal(rng, (N, r), 0.01))
    dy = bf16_bits(_normal(rng, (M, N), 1.0))
    return Workload(name=f"train linear W {N}x{K} bf16, M={M}, r={r}", W=W,
                    W_dtype="bf16", x=x, A=A, B=B, dy=dy, M=M, N=N, K=K, r=r,
                    alpha=alpha)


def decoder_layer_projection(targets, idx, std, seed):
    """bf16 N(0, std) weight of projection ``idx`` of one decoder layer.

    Each projection has its own generator, ``default_rng([seed, idx])``, so
    one projection can be drawn without drawing the others."""
    name, n, k = targets[idx]
    return bf16_bits(_normal(np.random.default_rng([seed, idx]), (n, k), std))


def decoder_layer_weights(targets, std, seed):
    """bf16 N(0, std) weights for every projection of one decoder layer."""
    return [(targets[i][0], decoder_layer_projection(targets, i, std, seed))
            for i in range(len(targets))]


def decoder_layer_linear(targets, idx, M, r, alpha, std, seed):
    """One projection of a decoder layer as a training-step linear: the
    weight of ``decoder_layer_projection``, then x [M, K], A [r, K], B [N, r]
    and dy [M, N] from ``default_rng([seed, 1000 + idx])`` (x, dy N(0, 1);
    A, B N(0, 0.01))."""
    name, N, K = targets[idx]
    W = decoder_layer_projection(targets, idx, std, seed)
    rng = np.random.default_rng([seed, 1000 + idx])
    x = bf16_bits(_normal(rng, (M, K), 1.0))
    A = bf16_bits(_normal(rng, (r, K), 0.01))
    B = bf16_bits(_normal(rng, (N, r), 0.01))
    dy = bf16_bits(_normal(rng, (M, N), 1.0))
    return Workload(name=f"{name} W {N}x{K} bf16 N(0,{std}), M={M}, r={r}", W=W,
                    W_dtype="bf16", x=x, A=A, B=B, dy=dy, M=M, N=N, K=K, r=r, alpha=alpha)
