"""Pins of oracle/codebooks.py: the FP4 table against the E2M1 format's own
bit-level definition, the FP4 quantiser against brute force with exact
rationals, the E4M3 encoder against torch's float8_e4m3fn conversion (an
independent implementation), the error bounds of both level-2 codes, and
the error study the pages' advice rests on; the mean-centred code against a
hand-worked group, brute-force nearest levels in exact rationals, the
pairing order of its sum, its half-step error bound and special cases."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codebooks, nf4


def e2m1_from_bits(bits):
    """Value of a 4-bit E2M1 pattern: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s, e, m = bits >> 3, (bits >> 1) & 3, bits & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if s else mag


def test_fp4_table_is_e2m1_over_6():
    q = codebooks.fp4_codebook()
    assert q.dtype == np.float32 and q.size == 16
    values = sorted({e2m1_from_bits(b) / 6 for b in range(16)})  # -0 == +0: 15 values
    assert len(values) == 15
    want = values[:8] + values[7:]  # zero entered twice
    assert np.all(np.diff(q) >= 0) and q[0] == -1 and q[15] == 1
    assert q[7].view(np.uint32) == 0 and q[8].view(np.uint32) == 0
    # each entry is the fp32 nearest to its exact value (1/12, 1/6, 1/3 and
    # 2/3 are not dyadic): within half an ulp, and exact where dyadic
    for v, fr in zip(q, want):
        err = abs(Fraction(float(v)) - fr)
        if fr == 0:
            assert err == 0
        else:
            assert err <= Fraction(float(np.spacing(np.float32(abs(float(fr)))))) / 2
        if fr.denominator & (fr.denominator - 1) == 0:
            assert err == 0


def brute_code(v, table):
    """Nearest entry with exact rationals, ties to the lower index."""
    fv = Fraction(float(v))
    dists = [abs(fv - Fraction(float(t))) for t in table]
    return min(range(16), key=lambda i: (dists[i], i))


def test_fp4_quantiser_against_brute_force():
    q = codebooks.fp4_codebook()
    vals = []
    for a, b in zip(q[:-1], q[1:]):
        mid = (float(a) + float(b)) / 2
        m32 = np.float32(mid)
        vals += [m32, np.nextafter(m32, np.float32(-2)), np.nextafter(m32, np.float32(2)), a, b]
    rng = np.random.default_rng(0)
    vals += list(rng.uniform(-1, 1, 300).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    vals = vals[np.abs(vals) <= 1]
    n = (vals.size // 63) * 63
    blocks = vals[:n].reshape(-1, 63)
    # one element of magnitude exactly 1 per block keeps v = fl32(w / 1) = w
    w = np.concatenate([blocks, np.ones((blocks.shape[0], 1), np.float32)], axis=1)
    packed, absmax = codebooks.quantize_4bit(w, "fp4")
    assert np.all(absmax == 1)
    codes = nf4.unpack_codes(packed, w.size).reshape(w.shape)
    for row, crow in zip(w, codes):
        for v, c in zip(row, crow):
            # the two equal zero entries make the code of a zero value
            # ambiguous; the value is not: compare what the code decodes to
            assert q[c] == q[brute_code(v, q)], (v, c)


def test_nf4_through_the_generic_quantiser_is_nf4():
    w = np.random.default_rng(1).standard_normal(64 * 50).astype(np.float32)
    w[:64] = 0
    p1, a1 = codebooks.quantize_4bit(w, "nf4")
    p2, a2 = nf4.quantize_nf4(w)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)


def test_fp4_zero_block_and_zero_weights_decode_to_plus_zero():
    w = np.zeros(128, np.float32)
    w[64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    w[70] = 0.0
    w[71] = -0.0
    packed, absmax = codebooks.quantize_4bit(w, "fp4")
    out = codebooks.dequantize_4bit(packed, absmax, 128, "fp4")
    assert np.all(out[:64].view(np.uint32) == 0)
    assert out[70].view(np.uint32) == 0 and out[71].view(np.uint32) == 0


def test_e4m3_encoder_matches_torch_float8():
    vals = codebooks.e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(500))])
    rng = np.random.default_rng(2)
    pts = np.concatenate([pts, rng.uniform(0, 1, 20000).astype(np.float32),
                          np.exp2(rng.uniform(-12, 8.8, 20000)).astype(np.float32)])
    pts = pts[(pts >= 0) & (pts <= 448)]
    ours = codebooks.e4m3_encode(pts.astype(np.float64))
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(codebooks.e4m3_values(),
                          torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn)
                          .to(torch.float64).numpy())


def test_fp8_double_quant_bounds():
    rng = np.random.default_rng(3)
    c = np.abs(rng.standard_normal(256 * 40)).astype(np.float32) * 0.05 + 1e-3
    c[5] = 0.0
    q, c2 = codebooks.double_quantize_fp8(c)
    cp = codebooks.dequant_scales_fp8(q, c2)
    g = np.arange(c.size) // 256
    # each group's maximum is stored exactly (ratio 1 = code 0x38), zero as 0
    for k in range(c2.size):
        i = k * 256 + int(np.argmax(c[k * 256:(k + 1) * 256]))
        assert q[i] == 0x38 and cp[i] == c[i]
    assert q[5] == 0 and cp[5] == 0
    # relative error of a normal E4M3 number: half a unit of the 3-bit mantissa
    ratio = c / c2[g]
    normal = ratio >= 2.0 ** -6
    err = np.abs(cp.astype(np.float64) - c)
    assert np.all(err[normal] <= 2.0 ** -4 * c[normal] * (1 + 2.0 ** -20))
    # the uint8 code: half a level, c2 / 510, plus fp32 rounding
    q8, c2u = nf4.double_quantize(c)
    cu = nf4.dequant_scales(q8, c2u)
    assert np.all(np.abs(cu.astype(np.float64) - c) <= c2u[g] / 510 * (1 + 2.0 ** -20) + 2.0 ** -24 * c)


def test_error_study_matches_the_pages_advice():
    """[kwkr] §2.2: NF4 suits normally distributed weights; §4.1: FP4 serves
    them worse.  Relative MSE over blocks of 64, absmax per block, no double
    quantisation.  The uniform INT4 grid of [czcl] §2.1 loses to NF4 on
    normal and heavy-tailed weights and wins on uniform ones, so the
    ordering comes from the weight distribution, not from the grids alone."""
    rng = np.random.default_rng(4)
    n = 64 * 8000
    dists = {"normal": rng.standard_normal(n), "student_t5": rng.standard_t(5, n),
             "uniform": rng.uniform(-1, 1, n)}
    res = {}
    for name, w in dists.items():
        w = w.astype(np.float32)
        row = {}
        for kind in ("nf4", "fp4"):
            p, a = codebooks.quantize_4bit(w, kind)
            row[kind] = codebooks.relative_mse(w, codebooks.dequantize_4bit(p, a, n, kind))
        row["int4"] = codebooks.relative_mse(w, codebooks.int4_uniform_roundtrip(w))
        res[name] = row
    for name in ("normal", "student_t5"):
        assert res[name]["nf4"] < res[name]["fp4"] < res[name]["int4"], res[name]
    assert res["uniform"]["int4"] < res["uniform"]["nf4"], res["uniform"]
    assert 0.007 < res["normal"]["nf4"] < 0.010


def test_uniform_int4_hand_worked_blocks():
    """The uniform strawman of [czcl] §2.1 on blocks whose levels are exact
    (absmax 7 * 2^e makes the level spacing the power of two 2^e), with the
    result of every value worked out by hand from the definition: nearest
    of the 15 levels j * absmax / 7, ties to the even j."""
    # absmax 7: levels are the integers -7..7
    blk = np.array([7.0, 3.5, -3.5, 2.5, -2.5, 0.5, -0.5, 6.6, -6.6, 1.2,
                    0.0, -7.0, 4.49, 4.51, -1.5, 1.5])
    want = np.array([7.0, 4.0, -4.0, 2.0, -2.0, 0.0, 0.0, 7.0, -7.0, 1.0,
                     0.0, -7.0, 4.0, 5.0, -2.0, 2.0])
    assert np.array_equal(codebooks.int4_uniform_roundtrip(blk, blocksize=16), want)
    # absmax 14 (spacing 2): 3 and 5 are half-way (1.5 and 2.5 steps) and take
    # the even levels 2 -> 4.0; 1 (half a step) goes to 0; -13 is 6.5 steps and
    # goes to -6 -> -12.0; 14 is the top level
    blk = np.array([14.0, 3.0, 5.0, 1.0, -13.0, -1.0, 9.0, 0.25])
    want = np.array([14.0, 4.0, 4.0, 0.0, -12.0, 0.0, 8.0, 0.0])
    assert np.array_equal(codebooks.int4_uniform_roundtrip(blk, blocksize=8), want)
    # a negative absmax element maps to the bottom level exactly
    blk = np.array([-0.875, 0.0625, 0.4375, 0.5])  # absmax 0.875 = 7/8, spacing 1/8
    want = np.array([-0.875, 0.0, 0.5, 0.5])       # 0.0625 = half a step -> 0; 3.5 -> 4 steps
    assert np.array_equal(codebooks.int4_uniform_roundtrip(blk, blocksize=4), want)
    # an all-zero block stays zero; blocks are independent of each other
    blk = np.concatenate([np.zeros(4), [7.0, 1.4, -2.6, 0.0]])
    want = np.concatenate([np.zeros(4), [7.0, 1.0, -3.0, 0.0]])
    assert np.array_equal(codebooks.int4_uniform_roundtrip(blk, blocksize=4), want)


def test_uniform_int4_has_fifteen_symmetric_levels():
    """Every reconstructed value is an integer multiple of absmax / 7 between
    -7 and 7 steps, both ends are reached by the block's extreme values, and
    a block and its negation give negated results (the grid is symmetric)."""
    rng = np.random.default_rng(12)
    w = rng.standard_normal(64 * 50)
    w_hat = codebooks.int4_uniform_roundtrip(w).reshape(-1, 64)
    blocks = w.reshape(-1, 64)
    step = np.abs(blocks).max(1, keepdims=True) / 7.0
    j = w_hat / step
    assert np.allclose(j, np.rint(j), atol=1e-9) and np.all(np.abs(np.rint(j)) <= 7)
    assert len(np.unique(np.rint(j))) <= 15
    k = np.argmax(np.abs(blocks), axis=1)
    assert np.allclose(np.abs(w_hat[np.arange(len(k)), k]), 7 * step[:, 0], rtol=1e-15)
    assert np.array_equal(codebooks.int4_uniform_roundtrip(-w), -codebooks.int4_uniform_roundtrip(w))
    # the error of every value is at most half a step
    assert np.all(np.abs(w_hat - blocks) <= step / 2 * (1 + 1e-12))


# ---- mean-centred double quantisation -------------------------------------

def test_centred_dq_hand_worked_group():
    """Constants 1, 2, 3, 6: mean 3, centred -2, -1, 0, 3, group max |d| = 3,
    t = -2/3, -1/3, 0, 1 -> nearest k / 127: 127 t = -84.67, -42.33, 0, 127
    -> k = -85, -42, 0, 127 (bytes 171, 214, 0, 127)."""
    q, c2, mu = codebooks.double_quantize_centred(np.array([1, 2, 3, 6], np.float32))
    assert mu == 3.0 and c2.tolist() == [3.0]
    assert q.tolist() == [171, 214, 0, 127]
    cp = codebooks.dequant_scales_centred(q, c2, mu)
    # c' = 3 + 3 k / 127 up to fp32 rounding: 0.99213, 2.00787, 3, 6
    want = [3 - 255 / 127, 3 - 126 / 127, 3.0, 6.0]
    assert np.allclose(cp.astype(np.float64), want, rtol=0, atol=4e-7)
    assert cp[2] == 3.0 and cp[3] == 6.0


def test_tree_sum_pairs_adjacent_values():
    """1 + 2^-53 rounds to 1 in fp64 (a tie, to even) but 2^-53 + 2^-53 is
    exact: adjacent pairing gives (1 + 2^-53) + (2^-53 + 2^-53) = 1 + 2^-52,
    where a left-to-right sum gives 1; five values pad to eight with zeros."""
    e = 2.0 ** -53
    assert codebooks.tree_sum_f64([1.0, e, e, e]) == 1.0 + 2.0 ** -52
    assert codebooks.tree_sum_f64([e, e, e, 1.0]) == 1.0 + 2.0 ** -52
    assert codebooks.tree_sum_f64([1.0, e, e, e, 0.5]) == 1.5 + 2.0 ** -52
    assert codebooks.tree_sum_f64([]) == 0.0 and codebooks.tree_sum_f64([2.5]) == 2.5
    # integers below 2^20: every order is exact, so the sum is the integer sum
    rng = np.random.default_rng(11)
    ints = rng.integers(0, 1 << 20, size=12345)
    assert codebooks.tree_sum_f64(ints.astype(np.float32)) == float(int(ints.sum()))


def test_centred_offset_is_the_mean():
    """mu is the mean of the constants to fp32 rounding (exact mean from
    math.fsum), so the centred constants average to about zero."""
    import math
    rng = np.random.default_rng(12)
    c = np.abs(rng.standard_normal((700, 64))).max(axis=1).astype(np.float32) * 0.02
    mu = codebooks.centred_offset(c)
    exact = math.fsum(c.astype(np.float64)) / c.size
    assert abs(float(mu) - exact) <= 2.0 ** -24 * exact * 1.0001
    d = (c - mu).astype(np.float64)
    assert abs(d.mean()) <= 2.0 ** -22 * exact


def test_s8_encode_is_the_nearest_level_by_brute_force():
    """Against exhaustive search over the 255 levels in exact rationals, ties
    toward k = 0, on random t, on every level and on every exact mid-point."""
    lv = [Fraction(float(codebooks._nearest_f32(Fraction(k, 127)))) for k in range(-127, 128)]
    rng = np.random.default_rng(13)
    ts = list(rng.uniform(-1, 1, 300).astype(np.float32))
    ts += [np.float32(float(v)) for v in lv]
    for j in range(127):
        m = (lv[127 + j] + lv[128 + j]) / 2
        f = np.float32(float(m))
        if Fraction(float(f)) == m:  # mid-points that are fp32 numbers are ties
            ts += [f, -f]
    ts = np.array(ts, dtype=np.float32)
    got = codebooks.s8_encode(ts).view(np.int8).astype(int)
    for t, k in zip(ts, got):
        ft = Fraction(float(t))
        dist = [abs(ft - v) for v in lv]
        best = min(dist)
        cands = [i - 127 for i, d in enumerate(dist) if d == best]
        assert k == min(cands, key=abs), (t, k, cands)
    # symmetry: -t takes the negated code
    assert np.array_equal(codebooks.s8_encode(-ts).view(np.int8), -got.astype(np.int8))


def test_s8_levels_are_k_over_127():
    """Byte b holds the fp32 nearest to k / 127 (k = b as a signed byte):
    both fp32 neighbours are farther from k / 127."""
    lv = codebooks.s8_levels()
    for b in range(256):
        k = b - 256 if b >= 128 else b
        f = lv[b]
        d = abs(Fraction(float(f)) - Fraction(k, 127))
        for nb in (np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))):
            assert abs(Fraction(float(nb)) - Fraction(k, 127)) > d, b
    assert lv[0] == 0 and lv[127] == 1 and lv[129] == -1


def test_centred_dq_error_is_half_a_level():
    """|c' - c| <= c2 / 254 (half a step of the group's signed grid) plus the
    fp32 roundings of d, t, the product and the sum."""
    rng = np.random.default_rng(14)
    w = rng.standard_normal((3000, 64)).astype(np.float32)
    c = np.abs(w).max(axis=1).astype(np.float32) * np.float32(0.02)
    q, c2, mu = codebooks.double_quantize_centred(c)
    cp = codebooks.dequant_scales_centred(q, c2, mu).astype(np.float64)
    g = np.arange(c.size) // 256
    slack = 2.0 ** -22 * (c.astype(np.float64) + c2[g] + float(mu))
    assert np.all(np.abs(cp - c) <= c2[g] / 254 + slack)


def test_centred_dq_special_cases():
    """Equal constants centre to zero: c2 = 0, every code 0, c' = mu = c
    exactly; one constant is its own mean; zero constants give mu = 0."""
    c = np.full(300, 0.0375, np.float32)
    q, c2, mu = codebooks.double_quantize_centred(c)
    assert mu == np.float32(0.0375) and not q.any() and not c2.any()
    assert np.array_equal(codebooks.dequant_scales_centred(q, c2, mu), c)
    q, c2, mu = codebooks.double_quantize_centred(np.array([0.7], np.float32))
    assert mu == np.float32(0.7) and q.tolist() == [0]
    q, c2, mu = codebooks.double_quantize_centred(np.zeros(5, np.float32))
    assert mu == 0 and not q.any() and not c2.any()


def test_level2_error_study():
    """Relative MSE of the block constants of normal weights (blocks of 64)
    under the three level-2 codes.  Centring pays: the constants of normal
    blocks cluster around their mean (about 2.5 sigma), so the signed grid's
    step, max |c - mu| / 127, is finer than the uint8 grid's max c / 255;
    without the centring the signed grid (max c / 127) would lose to it."""
    rng = np.random.default_rng(15)
    w = rng.standard_normal((8000, 64)).astype(np.float32)
    c = np.abs(w).max(axis=1).astype(np.float32)
    q8, c2 = nf4.double_quantize(c)
    mse_u8 = codebooks.relative_mse(c, nf4.dequant_scales(q8, c2))
    qf, cf = codebooks.double_quantize_fp8(c)
    mse_fp8 = codebooks.relative_mse(c, codebooks.dequant_scales_fp8(qf, cf))
    qc, cc, mu = codebooks.double_quantize_centred(c)
    mse_c = codebooks.relative_mse(c, codebooks.dequant_scales_centred(qc, cc, mu))
    assert mse_c < mse_u8 < mse_fp8, (mse_c, mse_u8, mse_fp8)
