"""The "4-bit storage, 16-bit compute" linear layer with a LoRA bypass, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Shapes (the torch Linear convention): W[N, K] (out_features x in_features),
x[M, K], A[r, K], B[N, r], y[M, N].  Inputs arrive as exact fp64 widenings
of the bf16 activations / LoRA matrices and of the fp32 dequantised weight.

  forward          y  = x W^T + s (x A^T) B^T                s = alpha / r
  backward (input) dx = dy W + s (dy B) A
  LoRA gradients   dA = s (dy B)^T x,   dB = s dy^T (x A^T)
  merge            W' = W + s B A

[rkmt] §2.1: the update is the product B A of a d x r and an r x k matrix,
with the frozen weight unchanged; [rkmt] §3.3: the low-rank update is scaled
by alpha / r.  ([czcl] §2.2 writes h = W0 x + B A x without the scale; the
scaled form is the reading taken.)  [kwkr] §2.3: gradients flow only into
the LoRA bypass; the 4-bit weight receives none, so there is no dW and no
gradient for the quantisation constants.  LoRA dropout is 0 and there is no
bias on this path (reading; [rkmt] §3.3 trains no bias).
A rank of 0 (or absent A/B) is the frozen layer.
"""

import numpy as np


def _scale(alpha, r):
    return 0.0 if r == 0 else float(alpha) / float(r)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lora_down(x, A):
    """u = x A^T  ([M, r])."""
    return _f64(x) @ _f64(A).T


def lora_up_input(dy, B):
    """t = dy B  ([M, r])."""
    return _f64(dy) @ _f64(B)


def linear_forward(x, w_hat, A, B, alpha, r):
    """y = x W^T + (alpha/r) (x A^T) B^T."""
    y = _f64(x) @ _f64(w_hat).T
    if r:
        y = y + _scale(alpha, r) * (lora_down(x, A) @ _f64(B).T)
    return y


def linear_backward_input(dy, w_hat, A, B, alpha, r):
    """dx = dy W + (alpha/r) (dy B) A."""
    dx = _f64(dy) @ _f64(w_hat)
    if r:
        dx = dx + _scale(alpha, r) * (lora_up_input(dy, B) @ _f64(A))
    return dx


def lora_grads(x, dy, A, B, alpha, r):
    """(dA, dB) = ((alpha/r) (dy B)^T x, (alpha/r) dy^T (x A^T)); no dW."""
    s = _scale(alpha, r)
    dA = s * (lora_up_input(dy, B).T @ _f64(x))
    dB = s * (_f64(dy).T @ lora_down(x, A))
    return dA, dB


def lora_merge(w_hat, A, B, alpha, r):
    """W' = W + (alpha/r) B A in fp64 ([N, K]).

    [rkmt] §2.1: for inference the adapter is folded into the weight,
    W <- W + B A, which adds no latency; [tgd] §7: a QLoRA adapter is merged
    into a 16-bit weight, never into the 4-bit form.  Reading: the weight is
    the dequantised W the adapter was trained against (the value every
    forward of this layer used), scaled update as in the forward.
    """
    w = _f64(w_hat)
    if r:
        w = w + _scale(alpha, r) * (_f64(B) @ _f64(A))
    return w
