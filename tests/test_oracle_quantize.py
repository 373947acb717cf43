"""Pins for the oracle's level-1 NF4 quantiser and packing (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codebooks, nf4


def rn_f32(fr):
    """Exact rational -> nearest binary32 (ties to even, subnormals kept)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def brute_force_codes(w, blocksize=64):
    """Nearest table entry by exhaustive search in exact rationals.

    Absmax by Python's max over exact values; the normalised value is the
    exactly rounded fp32 quotient; ties go to the lower index.
    """
    table = [Fraction(float(t)) for t in nf4.nf4_codebook()]
    w = [Fraction(float(v)) for v in np.asarray(w, np.float32).ravel()]
    codes, absmax = [], []
    for b in range(0, len(w), blocksize):
        blk = w[b:b + blocksize]
        c = max(abs(v) for v in blk)
        absmax.append(c)
        for v in blk:
            if c == 0:
                codes.append(7)
                continue
            q = rn_f32(v / c)
            dists = [abs(q - t) for t in table]
            best = min(dists)
            codes.append(dists.index(best))  # lowest index on ties
    return np.array(codes, np.uint8), absmax


def pack_ref(codes):
    codes = [int(c) for c in codes]
    return np.array([(codes[i] << 4) | codes[i + 1] for i in range(0, len(codes), 2)],
                    np.uint8)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force_on_random_blocks(seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(64 * 5) * 0.02).astype(np.float32)
    w[70] = 0.0
    w[130:194] = 0.0  # one whole zero block
    packed, absmax = nf4.quantize_nf4(w)
    codes, amax = brute_force_codes(w)
    assert np.array_equal(packed, pack_ref(codes))
    assert [Fraction(float(a)) for a in absmax] == amax


def test_tiny_and_subnormal_scales_match_brute_force():
    """Blocks whose absmax is tiny (1e-30), at the bottom of the normal range
    (near 2^-126) or subnormal (1e-40, 1e-44, the smallest subnormal 2^-149),
    and blocks where w / c itself is subnormal or underflows to zero: the
    fp32 quotient and the nearest code follow the exact-rational brute force
    (IEEE division with gradual underflow, ties to the lower code)."""
    rng = np.random.default_rng(21)
    blocks = []
    for scale in (1e-30, 1.5e-38, 1e-40, 1e-44):
        b = (rng.standard_normal(64) * scale).astype(np.float32)
        blocks.append(b)
    tiny = np.zeros(64, np.float32)
    tiny[0] = np.float32(2.0 ** -149)     # absmax = the smallest subnormal
    tiny[1] = -np.float32(2.0 ** -149)    # v = -1 exactly
    blocks.append(tiny)
    mixed = np.zeros(64, np.float32)
    mixed[0] = np.float32(1.0)
    mixed[1:8] = np.array([1e-40, -1e-40, 2.0 ** -149, 1e-45, -3e-39, 1e-38, 5e-39], np.float32)
    mixed[8:64] = (rng.standard_normal(56) * 1e-3).astype(np.float32)
    blocks.append(mixed)
    big = (rng.standard_normal(64) * 1e30).astype(np.float32)  # large but finite
    blocks.append(big)
    w = np.concatenate(blocks)
    packed, absmax = nf4.quantize_nf4(w)
    codes, amax = brute_force_codes(w)
    assert np.array_equal(packed, pack_ref(codes))
    assert [Fraction(float(a)) for a in absmax] == amax
    assert absmax[4] == np.float32(2.0 ** -149)
    got = nf4.unpack_codes(packed)
    assert got[4 * 64] == 15 and got[4 * 64 + 1] == 0   # +-c of the subnormal block


def test_heavy_tailed_and_ragged_tail():
    rng = np.random.default_rng(7)
    w = (rng.standard_t(5, size=64 * 3 + 10) * 0.0155).astype(np.float32)
    packed, absmax = nf4.quantize_nf4(w)
    codes, amax = brute_force_codes(w)
    assert packed.size == w.size // 2 and absmax.size == 4
    assert np.array_equal(packed, pack_ref(codes))
    assert [Fraction(float(a)) for a in absmax] == amax


def test_absmax_element_gets_an_end_code():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 8) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize_nf4(w)
    codes = nf4.unpack_codes(packed)
    for b in range(8):
        blk = w[64 * b:64 * b + 64]
        k = int(np.argmax(np.abs(blk)))
        assert codes[64 * b + k] == (15 if blk[k] > 0 else 0)


def test_codes_on_the_grid_round_trip():
    q = nf4.nf4_codebook()
    c = np.float32(0.5)  # power of two: q*c is exact
    w = (q * c).astype(np.float32)
    w = np.concatenate([w, np.zeros(48, np.float32)])
    codes = nf4.unpack_codes(nf4.quantize_nf4(w)[0])
    assert list(codes[:16]) == list(range(16))


def test_ties_go_to_the_lower_code():
    # With c = 1 the normalised value is w itself.  For each mid-point either
    # it is an fp32 value (then it must take the lower code) or the fp32
    # values on either side of it must split between the two codes.
    mids = nf4.nf4_midpoints()
    for i, m in enumerate(mids):
        lo = np.float32(m)
        if float(lo) > m:
            lo = np.nextafter(lo, np.float32(-2))
        hi = np.nextafter(lo, np.float32(2))
        w = np.zeros(64, np.float32)
        w[0] = 1.0
        w[1], w[2] = lo, hi
        codes = nf4.unpack_codes(nf4.quantize_nf4(w)[0])
        if float(lo) == m:
            assert codes[1] == i, "exact mid-point must take the lower code"
        else:
            assert codes[1] == i
        assert codes[2] == i + 1


def test_zero_block_and_negative_zero():
    w = np.zeros(128, np.float32)
    w[64:] = -0.0
    packed, absmax = nf4.quantize_nf4(w)
    assert np.all(absmax == 0)
    assert np.all(nf4.unpack_codes(packed) == 7)
    w2 = np.zeros(64, np.float32)
    w2[0] = 0.5
    w2[1] = -0.0
    assert nf4.unpack_codes(nf4.quantize_nf4(w2)[0])[1] == 7


def test_nibble_order_even_element_high():
    w = np.zeros(64, np.float32)
    w[0], w[1] = 1.0, -1.0
    packed, _ = nf4.quantize_nf4(w)
    assert packed[0] == 0xF0


def test_division_not_reciprocal_multiply():
    # Find inputs where fl32(w * fl32(1/c)) and fl32(w / c) fall on
    # different sides of a threshold; the oracle must follow the division.
    rng = np.random.default_rng(11)
    mids = nf4.nf4_midpoints()
    found = 0
    for _ in range(4000):
        c = np.float32(rng.uniform(0.01, 0.1))
        i = int(rng.integers(0, 15))
        base = np.float32(mids[i] * float(c))
        for k in range(-40, 41):
            w = np.float32(base + np.float32(k) * np.spacing(base))
            q_div = np.float32(w / c)
            q_rcp = np.float32(w * np.float32(np.float32(1.0) / c))
            if (q_div > mids[i]) != (q_rcp > mids[i]):
                blk = np.zeros(64, np.float32)
                blk[0], blk[1] = c, w
                code = nf4.unpack_codes(nf4.quantize_nf4(blk)[0])[1]
                exact = brute_force_codes(blk)[0][1]
                assert code == exact
                found += 1
                break
        if found >= 5:
            break
    assert found >= 1


def test_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(5)
    w32 = (rng.standard_normal(256) * 0.02).astype(np.float32)
    bits = nf4.f32_to_bf16_bits(w32)
    wbf = nf4.bf16_bits_to_f32(bits)
    packed, absmax = nf4.quantize_nf4(wbf)
    codes, amax = brute_force_codes(wbf)
    assert np.array_equal(packed, pack_ref(codes))


def test_blocks_are_independent():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(64 * 4) * 0.02).astype(np.float32)
    p1, a1 = nf4.quantize_nf4(w)
    w2 = w.copy()
    w2[64:128] *= 100
    p2, a2 = nf4.quantize_nf4(w2)
    assert np.array_equal(p1[:32], p2[:32]) and np.array_equal(p1[64:], p2[64:])
    assert a1[0] == a2[0] and np.array_equal(a1[2:], a2[2:])


def test_nf4_beats_uniform_int4_on_normal_weights():
    # [kwkr] §2.1-2.2: a uniform 16-level grid wastes levels on normal data;
    # the quantile grid loses less.  The uniform baseline is the oracle's
    # symmetric 15-level strawman of [czcl] §2.1 (pinned by hand-worked
    # blocks in test_oracle_codebooks.py).
    rng = np.random.default_rng(0)
    w = (rng.standard_normal(64 * 4096) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize_nf4(w)
    w_nf4 = nf4.dequantize(packed, absmax, w.size)
    w_int4 = codebooks.int4_uniform_roundtrip(w)
    mse_nf4 = np.mean((w_nf4 - w) ** 2)
    mse_int4 = np.mean((w_int4 - w) ** 2)
    assert mse_nf4 < mse_int4


def test_rejects_odd_and_nonfinite():
    with pytest.raises(ValueError):
        nf4.quantize_nf4(np.zeros(3, np.float32))
    with pytest.raises(ValueError):
        nf4.quantize_nf4(np.array([np.inf, 0], np.float32))
