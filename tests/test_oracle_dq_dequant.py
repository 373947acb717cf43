"""Pins for the oracle's double quantisation and dequantisation (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import memory, nf4
from tests.test_oracle_quantize import rn_f32


def brute_force_dq(c, group=256):
    """Nearest 8-bit level by exhaustive search in exact rationals."""
    levels = [Fraction(float(v)) for v in nf4.dq_levels()]
    c = [Fraction(float(v)) for v in np.asarray(c, np.float32)]
    q, c2 = [], []
    for g in range(0, len(c), group):
        grp = c[g:g + group]
        m = max(grp)
        c2.append(m)
        for v in grp:
            if m == 0:
                q.append(0)
                continue
            t = rn_f32(v / m)
            d = [abs(t - l) for l in levels]
            q.append(d.index(min(d)))
    return np.array(q, np.uint8), c2


def test_levels_are_the_unsigned_unit_grid():
    lv = nf4.dq_levels()
    assert lv.dtype == np.float32 and lv.shape == (256,)
    assert lv[0] == 0.0 and lv[255] == 1.0
    for q in (1, 7, 128, 254):
        assert Fraction(float(lv[q])) == rn_f32(Fraction(q, 255))


@pytest.mark.parametrize("seed", [0, 1])
def test_dq_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    c = np.abs(rng.standard_normal(256 * 2 + 37) * 0.05).astype(np.float32)
    c[5] = 0.0
    q8, c2 = nf4.double_quantize(c)
    qb, c2b = brute_force_dq(c)
    assert np.array_equal(q8, qb)
    assert [Fraction(float(v)) for v in c2] == c2b
    assert c2.size == 3


def test_group_max_gets_top_code_and_exact_scale():
    rng = np.random.default_rng(2)
    c = np.abs(rng.standard_normal(1024) * 0.05).astype(np.float32)
    q8, c2 = nf4.double_quantize(c)
    cp = nf4.dequant_scales(q8, c2)
    for g in range(4):
        k = 256 * g + int(np.argmax(c[256 * g:256 * g + 256]))
        assert q8[k] == 255
        assert cp[k] == c2[g] == c[k]


def test_dq_error_is_at_most_half_a_level():
    rng = np.random.default_rng(4)
    c = np.abs(rng.standard_t(5, 4096) * 0.05).astype(np.float32)
    q8, c2 = nf4.double_quantize(c)
    cp = nf4.dequant_scales(q8, c2).astype(np.float64)
    step = np.repeat(c2.astype(np.float64), 256) / 255.0
    assert np.all(np.abs(cp - c) <= step / 2 * (1 + 1e-6) + 1e-12)


def test_zero_group():
    q8, c2 = nf4.double_quantize(np.zeros(300, np.float32))
    assert np.all(q8 == 0) and np.all(c2 == 0)


def test_storage_bits_per_parameter():
    # Scale memory falls from 32/64 to 8/64 + 32/(64*256) bit per weight.
    assert memory.bits_per_param(double_quant=False) == 4.5
    assert memory.bits_per_param() == 4 + 8 / 64 + 32 / (64 * 256)
    assert abs(memory.bits_per_param() - 4.126953125) < 1e-12
    assert abs(memory.dq_saving_bits() - 0.373046875) < 1e-12


def test_code_seven_dequantises_to_exact_positive_zero():
    packed = np.full(32, 0x77, np.uint8)
    out = nf4.dequantize(packed, np.array([0.37], np.float32), 64)
    assert np.all(out.view(np.uint32) == 0)


def test_outlier_group_gives_signed_zero_blocks():
    # A group whose max dwarfs a block constant drives its 8-bit code to 0;
    # then c' = 0 and negative codes dequantise to -0.0 (IEEE product).
    c = np.full(256, 1e-6, np.float32)
    c[0] = 10.0
    q8, c2 = nf4.double_quantize(c)
    assert q8[1] == 0
    cp = nf4.dequant_scales(q8, c2)
    packed = np.full(32, 0x07, np.uint8)  # codes 0 and 7 alternating
    out = nf4.dequantize(packed, cp[1:2], 64)
    assert out.view(np.uint32)[0] == 0x80000000  # -0.0 from code 0
    assert out.view(np.uint32)[1] == 0


def _pipeline(w):
    packed, absmax = nf4.quantize_nf4(w)
    q8, c2 = nf4.double_quantize(absmax)
    cp = nf4.dequant_scales(q8, c2)
    return packed, absmax, q8, c2, nf4.dequantize(packed, cp, w.size)


@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_quantisation_is_idempotent_with_double_quant(dist):
    rng = np.random.default_rng(12)
    n = 64 * 256 * 3
    if dist == "normal":
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    else:
        w = (rng.standard_t(5, n) * 0.0155).astype(np.float32)
    p1, _, q1, c21, w1 = _pipeline(w)
    p2, _, q2, c22, w2 = _pipeline(w1)
    assert np.array_equal(q1, q2)
    assert np.array_equal(c21.view(np.uint32), c22.view(np.uint32))
    live = np.repeat(q1 > 0, 32)
    assert np.array_equal(p1[live], p2[live])
    assert np.array_equal(w1, w2)  # IEEE ==: only +-0 may differ in bits


def test_quantisation_is_idempotent_without_double_quant():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal(64 * 100) * 0.02).astype(np.float32)
    p1, a1 = nf4.quantize_nf4(w)
    w1 = nf4.dequantize(p1, a1, w.size)
    p2, a2 = nf4.quantize_nf4(w1)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
    assert np.array_equal(nf4.dequantize(p2, a2, w.size).view(np.uint32), w1.view(np.uint32))


def test_dequant_error_bound():
    # Each weight lands within half of the widest code gap of its block scale.
    rng = np.random.default_rng(14)
    w = (rng.standard_normal(64 * 64) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize_nf4(w)
    wq = nf4.dequantize(packed, absmax, w.size).astype(np.float64)
    gap = np.max(np.diff(nf4.nf4_codebook().astype(np.float64)))
    bound = np.repeat(absmax.astype(np.float64), 64) * gap / 2 * (1 + 1e-6)
    assert np.all(np.abs(wq - w) <= bound)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.0078125 + 2 ** -10, -0.0, 3.0e-39, 1.01171875],
                 np.float32)
    bits = nf4.f32_to_bf16_bits(x)
    want = [0x3F80, 0x3F80, 0x3F81, 0x8000, 0x0021, 0x3F82]
    assert list(bits) == want
