"""Pins of oracle/codebooks.py: the FP4 table against the E2M1 format's own
bit-level definition, the FP4 quantiser against brute force with exact
rationals, the E4M3 encoder against torch's float8_e4m3fn conversion (an
independent implementation), the error bounds of both level-2 codes, and
the error study the pages' advice rests on."""

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
