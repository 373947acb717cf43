"""Pins of oracle/dropout.py against things other than itself: numpy's own
Philox bit generator (an independent implementation of the published
Philox4x64-10), the statistics a dropout mask must have, and the adjoint
identities of the dropped adapter branch."""

import numpy as np
import pytest

from oracle import dropout, linear

U64 = (1 << 64) - 1


def numpy_block(c, key):
    """The Philox4x64-10 block at counter c (4 words) from numpy's generator,
    which advances its counter by one before each block."""
    prev = list(c)
    i = 0
    while prev[i] == 0:       # counter - 1 with borrow
        prev[i] = U64
        i += 1
    prev[i] -= 1
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


@pytest.mark.parametrize("c,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((6, 0, 0, 0), (7, 9)),
    ((U64, U64, U64, U64), (U64, U64)),
    ((0, 1, 0, 0), (0x243F6A8885A308D3, 0x13198A2E03707344)),
    ((123456789, 987654321, 5, 77), (2**63 + 11, 3)),
])
def test_philox_matches_numpys_generator(c, key):
    out = dropout.philox4x64_10(*[np.uint64(v) for v in c], key[0], key[1])
    assert [int(np.asarray(w)) for w in out] == numpy_block(c, key)


def test_philox_on_random_counters_and_keys():
    rng = np.random.default_rng(0)
    for _ in range(20):
        c = [int(v) for v in rng.integers(0, 2**64, size=4, dtype=np.uint64)]
        key = [int(v) for v in rng.integers(0, 2**64, size=2, dtype=np.uint64)]
        if c == [0, 0, 0, 0]:
            continue
        out = dropout.philox4x64_10(*[np.uint64(v) for v in c], key[0], key[1])
        assert [int(np.asarray(w)) for w in out] == numpy_block(c, key)


def test_mask_layout_from_numpys_stream():
    """Each 8-row group of a column reads the 8 32-bit halves of one block,
    low half first, compared with floor(p 2^32)."""
    M, K, p, seed = 24, 10, 0.3, 1234567
    keep = dropout.dropout_keep(M, K, p, seed)
    thr = int(np.floor(float(np.float32(p)) * 2**32))
    for k in range(K):
        for b in range(M // 8):
            if k == 0 and b == 0:
                words = [int(np.asarray(w)) for w in dropout.philox4x64_10(
                    np.uint64(0), np.uint64(0), np.uint64(0), np.uint64(0), seed, 0)]
                # counter 0 has no predecessor in numpy's stream: it is the
                # successor of the all-ones counter, which wraps to zero
                assert words == numpy_block_wrapped(seed)
            else:
                words = numpy_block((k, b, 0, 0), (seed, 0))
            halves = []
            for w in words:
                halves += [w & 0xFFFFFFFF, w >> 32]
            assert [h >= thr for h in halves] == list(keep[8 * b:8 * b + 8, k])


def numpy_block_wrapped(seed):
    bg = np.random.Philox(counter=np.array([U64] * 4, dtype=np.uint64),
                          key=np.array([seed, 0], dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


def test_threshold_edges():
    assert dropout.keep_threshold(0.0) == 0
    assert dropout.keep_threshold(0.5) == 2**31
    assert dropout.keep_threshold(0.25) == 2**30
    assert dropout.dropout_keep(16, 64, 0.0, 5).all()
    with pytest.raises(ValueError):
        dropout.keep_threshold(1.0)
    with pytest.raises(ValueError):
        dropout.keep_threshold(-0.1)


@pytest.mark.parametrize("p", [0.05, 0.1, 0.5])
def test_mask_statistics(p):
    M, K = 512, 640
    keep = dropout.dropout_keep(M, K, p, seed=42)
    n = keep.size
    drop = 1.0 - keep.mean()
    assert abs(drop - p) < 5 * np.sqrt(p * (1 - p) / n)
    # every row residue mod 8 (every 32-bit half) drops at rate p
    for j in range(8):
        d = 1.0 - keep[j::8].mean()
        assert abs(d - p) < 5 * np.sqrt(p * (1 - p) / (n / 8))
    # neighbouring rows and columns are independent: agreement p^2 + (1-p)^2
    agree = 1 - p * (2 - 2 * p)
    for a, b in ((keep[:-1], keep[1:]), (keep[:, :-1], keep[:, 1:])):
        got = (a == b).mean()
        assert abs(got - agree) < 5 * np.sqrt(agree * (1 - agree) / a.size)


def test_mask_is_a_function_of_seed_and_position():
    a = dropout.dropout_keep(64, 128, 0.1, 7)
    assert np.array_equal(a, dropout.dropout_keep(64, 128, 0.1, 7))
    assert not np.array_equal(a, dropout.dropout_keep(64, 128, 0.1, 8))
    big = dropout.dropout_keep(96, 256, 0.1, 7)
    assert np.array_equal(big[:64, :128], a)


def test_dropped_input_is_unbiased():
    """E[x * keep / (1 - p)] = x: the mean over many seeds converges to x."""
    p = 0.25
    x = np.random.default_rng(3).standard_normal((8, 64))
    acc = np.zeros_like(x)
    S = 400
    for s in range(S):
        acc += dropout.lora_dropout(x, p, s)
    sd = np.abs(x) * np.sqrt(p / (1 - p) / S)
    assert np.all(np.abs(acc / S - x) < 5 * sd + 1e-12)
    xd = dropout.lora_dropout(x, p, 0)
    kept = xd != 0
    assert np.allclose(xd[kept], x[kept] / (1 - p), rtol=1e-15)


def test_zero_rate_is_the_plain_layer():
    rng = np.random.default_rng(4)
    M, N, K, r, alpha = 8, 64, 128, 4, 8.0
    x, dy = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    w = rng.standard_normal((N, K))
    A, B = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    y, u = dropout.linear_forward(x, w, A, B, alpha, r, 0.0, 9)
    assert np.array_equal(y, linear.linear_forward(x, w, A, B, alpha, r))
    dx, t = dropout.linear_backward_input(dy, w, A, B, alpha, r, 0.0, 9)
    assert np.array_equal(dx, linear.linear_backward_input(dy, w, A, B, alpha, r))


def test_adjoint_of_the_dropped_branch():
    """With W = 0 the layer is the linear map x -> s ((x D) A^T) B^T; its
    backward must be the adjoint: <dy, y(x)> = <dx(dy), x>.  A mask missing
    from either side, transposed, or on the wrong operand breaks it."""
    rng = np.random.default_rng(5)
    M, N, K, r, alpha, p, seed = 16, 64, 192, 8, 16.0, 0.3, 77
    x, dy = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    A, B = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    w0 = np.zeros((N, K))
    y, u = dropout.linear_forward(x, w0, A, B, alpha, r, p, seed)
    dx, t = dropout.linear_backward_input(dy, w0, A, B, alpha, r, p, seed)
    lhs, rhs = np.sum(dy * y), np.sum(dx * x)
    assert abs(lhs - rhs) <= 1e-11 * (np.sum(np.abs(dy * y)) + 1.0)
    # the check has teeth: the undropped backward fails it
    dx_plain = linear.linear_backward_input(dy, w0, A, B, alpha, r)
    assert abs(np.sum(dx_plain * x) - lhs) > 1e-3 * abs(lhs)


def test_lora_gradients_take_the_dropped_input():
    """y is linear in A and in B, so <dA, dA'> = <dy, y(dA')> and
    <dB, dB'> = <dy, y(dB')> exactly, with dA, dB from the dropped input."""
    rng = np.random.default_rng(6)
    M, N, K, r, alpha, p, seed = 16, 64, 128, 8, 16.0, 0.2, 3
    x, dy = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    A, B = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    w0 = np.zeros((N, K))
    dA, dB = linear.lora_grads(dropout.lora_dropout(x, p, seed), dy, A, B, alpha, r)
    dA2, dB2 = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    yA, _ = dropout.linear_forward(x, w0, dA2, B, alpha, r, p, seed)
    yB, _ = dropout.linear_forward(x, w0, A, dB2, alpha, r, p, seed)
    assert np.isclose(np.sum(dA * dA2), np.sum(dy * yA), rtol=1e-11)
    assert np.isclose(np.sum(dB * dB2), np.sum(dy * yB), rtol=1e-11)
