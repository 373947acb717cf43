"""Pins for the oracle's NF4 codebook (CPU only).

Each check ties the table to a property the pages state or to an independent
closed form, so that a dropped term, a wrong index or a wrong normaliser in
``oracle.nf4.nf4_codebook_f64`` fails at least one of them.
"""

import math
from fractions import Fraction

import numpy as np
import scipy.special as sps

from oracle import nf4


def test_sixteen_monotone_codes_with_exact_zero_and_unit_ends():
    # [rkmt] §2.2.1: 4 bits give 16 values; [czcl] §2.1: zero is exact.
    q = nf4.nf4_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    bits = q.view(np.uint32)
    assert bits[0] == np.float32(-1.0).view(np.uint32)
    assert bits[7] == 0  # +0.0, not -0.0
    assert bits[15] == np.float32(1.0).view(np.uint32)
    assert int(np.sum(q < 0)) == 7 and int(np.sum(q > 0)) == 8


def test_codes_are_equal_area_normal_quantiles():
    # [kwkr] §2.2: code points are standard-normal quantiles;
    # [rkmt] §2.2.1: the quantiles cut the truncated density into equal areas.
    # Checked with the forward CDF (scipy's ndtr) and scipy's own inverse
    # (ndtri) for the normaliser: a different routine from the oracle's.
    q = nf4.nf4_codebook_f64()
    p_max = float(nf4.P_MAX)
    top = sps.ndtri(p_max)
    for j in range(1, 9):
        want = 0.5 + (p_max - 0.5) * j / 8
        assert abs(sps.ndtr(q[7 + j] * top) - want) < 1e-14
    for j in range(1, 8):
        want = 0.5 + (p_max - 0.5) * j / 7
        assert abs(sps.ndtr(-q[7 - j] * top) - want) < 1e-14


def test_codes_match_closed_form_to_a_few_ulp():
    q = nf4.nf4_codebook_f64()
    p_max = float(nf4.P_MAX)
    top = sps.ndtri(p_max)
    want = ([-sps.ndtri(0.5 + (p_max - 0.5) * j / 7) / top for j in range(7, 0, -1)]
            + [0.0]
            + [sps.ndtri(0.5 + (p_max - 0.5) * j / 8) / top for j in range(1, 9)])
    for a, b in zip(q, want):
        # two independent inverse CDFs and a rounded probability: allow 8 ulp
        assert abs(a - b) <= 8 * np.spacing(abs(b)) + 1e-300


def test_dense_near_zero_sparse_in_tails():
    # [kwkr] §2.2: points are dense in the middle and sparse in the tails.
    q = nf4.nf4_codebook_f64()
    pos_gaps = np.diff(q[7:])
    neg_gaps = np.diff(q[:8])[::-1]
    assert np.all(np.diff(pos_gaps) > 0)
    assert np.all(np.diff(neg_gaps) > 0)


def test_truncation_point_value():
    # The one constant from outside the pages: 1 - (1/32 + 1/30)/2.
    assert nf4.P_MAX == Fraction(929, 960)
    assert math.isclose(float(nf4.P_MAX), 0.9677083333333333, rel_tol=0, abs_tol=1e-16)


def test_midpoints_exact_and_between_codes():
    q = nf4.nf4_codebook().astype(np.float64)
    m = nf4.nf4_midpoints()
    assert m.shape == (15,)
    for i in range(15):
        # exactness: 2*m reproduces the fp64 sum, which is exact for two fp32
        assert Fraction(m[i]) == (Fraction(float(q[i])) + Fraction(float(q[i + 1]))) / 2
        assert q[i] < m[i] < q[i + 1]
