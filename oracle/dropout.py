"""LoRA dropout on the adapter branch, fp64, with its counter-based mask.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[rkmt] §3.3 configures the LoRA layer with a dropout rate of 0.1 (to fight
overfitting); [czcl] §3.2 and [kwkr] §4 use 0.05.  The pages do not say where
the dropout sits.  Reading: it is the LoRA layer's own dropout, applied to the
input of the adapter branch only,

    y = x W^T + (alpha/r) ((x * D) A^T) B^T,     D = keep / (1 - p),

so the frozen base path sees the undropped x.  By the chain rule the
backward to the input is  dx = dy W + D * ((alpha/r) (dy B) A)  and the LoRA
gradients take the dropped input:  dA = (alpha/r) (dy B)^T (x * D),
dB = (alpha/r) dy^T ((x * D) A^T).

The mask must be regenerated in the backward pass without storing it, so it
comes from a counter-based generator: Philox4x64-10 (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), the 4-word,
64-bit-lane variant with ten rounds.  The mask layout is this library's own
convention (the pages have none):

  element (m, k) of a row-major [M, K] input uses the Philox block with
  counter (k, m // 8, 0, 0) and key (seed, 0); of its four 64-bit outputs it
  takes word (m % 8) // 2, low 32 bits for even m % 8, high 32 bits for odd;
  the element is kept iff that 32-bit value >= floor(p * 2^32).

so one block serves eight consecutive rows of one column.  p is the fp32
value the caller passes, widened exactly; the threshold is computed exactly in
fp64.
"""

import numpy as np

_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

# Philox4x64 round multipliers and key (Weyl) increments, as published
_MUL = (np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157))
_WEYL = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B))


def _mulhilo(a, b):
    """Full 128-bit product of 64-bit words as (high, low), from 32-bit limbs."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.uint64(b)
    a0, a1 = a & _M32, a >> _S32
    b0, b1 = b & _M32, b >> _S32
    ll = a0 * b0
    lh = a0 * b1
    hl = a1 * b0
    hh = a1 * b1
    carry = ((ll >> _S32) + (lh & _M32) + (hl & _M32)) >> _S32
    hi = hh + (lh >> _S32) + (hl >> _S32) + carry
    with np.errstate(over="ignore"):
        lo = a * b
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64 with ten rounds on arrays of counters; returns the 4 output words.

    A round multiplies counter words 0 and 2 by the two multipliers and
    mixes the high halves with words 1 and 3 and the key; the key takes its
    Weyl increment between rounds.
    """
    c = [np.asarray(v, dtype=np.uint64) for v in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c = [v.copy() for v in c]
    k0, k1 = np.uint64(k0), np.uint64(k1)
    for rnd in range(10):
        if rnd:
            with np.errstate(over="ignore"):
                k0 = np.uint64(k0 + _WEYL[0])
                k1 = np.uint64(k1 + _WEYL[1])
        hi0, lo0 = _mulhilo(c[0], _MUL[0])
        hi1, lo1 = _mulhilo(c[2], _MUL[1])
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def keep_threshold(p):
    """floor(p * 2^32) for the fp32 rate p in [0, 1)."""
    p = float(np.float32(p))
    if not 0.0 <= p < 1.0:
        raise ValueError("oracle: dropout rate must lie in [0, 1)")
    return int(np.floor(p * 4294967296.0))


def dropout_keep(M, K, p, seed):
    """Boolean keep mask [M, K] of the layout in the module docstring."""
    thr = keep_threshold(p)
    m = np.arange(M, dtype=np.uint64)[:, None]
    k = np.arange(K, dtype=np.uint64)[None, :]
    words = philox4x64_10(k, m >> np.uint64(3), 0, 0, np.uint64(seed), 0)
    j = (np.arange(M) % 8)[:, None] + np.zeros((1, K), dtype=np.int64)
    w64 = np.choose(j // 2, words)
    w32 = np.where(j % 2 == 0, w64 & _M32, w64 >> _S32)
    return w32 >= np.uint64(thr)


def lora_dropout(x, p, seed):
    """The adapter branch's input x * keep / (1 - p), fp64 ([rkmt] §3.3)."""
    x = np.asarray(x, dtype=np.float64)
    keep = dropout_keep(x.shape[0], x.shape[1], p, seed)
    return np.where(keep, x / (1.0 - float(np.float32(p))), 0.0)


def linear_forward(x, w_hat, A, B, alpha, r, p, seed):
    """y = x W^T + (alpha/r) ((x D) A^T) B^T; also returns u = (x D) A^T."""
    x = np.asarray(x, dtype=np.float64)
    xd = lora_dropout(x, p, seed)
    u = xd @ np.asarray(A, dtype=np.float64).T
    y = x @ np.asarray(w_hat, dtype=np.float64).T + (alpha / r) * (u @ np.asarray(B, dtype=np.float64).T)
    return y, u


def linear_backward_input(dy, w_hat, A, B, alpha, r, p, seed):
    """dx = dy W + D * ((alpha/r) (dy B) A); also returns t = dy B."""
    dy = np.asarray(dy, dtype=np.float64)
    t = dy @ np.asarray(B, dtype=np.float64)
    keep = dropout_keep(dy.shape[0], np.asarray(A).shape[1], p, seed)
    lora = (alpha / r) * (t @ np.asarray(A, dtype=np.float64))
    dx = dy @ np.asarray(w_hat, dtype=np.float64) + np.where(keep, lora / (1.0 - float(np.float32(p))), 0.0)
    return dx, t
