"""NF4 codebook, blockwise absmax quantisation, double quantisation, dequant.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Readings of the pages taken here (each is listed in the design doc as well):
  * Codebook: 7 negative normal quantiles, an exact 0 and 8 positive normal
    quantiles of a normal distribution truncated at probability P_MAX, all
    divided by the largest so the table spans [-1, 1] with 0 at index 7.
    The pages give the principle (quantiles of a normal, dense near 0,
    exact zero kept) but print no table and no truncation point; P_MAX is
    the single constant taken from outside the pages.
  * Level-1 quantisation: blocks of 64 consecutive weights of the row-major
    flattened tensor; constant = max |w| in fp32; v = fl32(w / c) by IEEE
    fp32 division; code = index of the nearest table entry, ties to the
    lower index (equivalently: the number of fp64 mid-points strictly below
    v); two codes per byte, the even element in the high nibble.
  * Double quantisation: groups of 256 consecutive block constants; group
    constant = fp32 max; v = fl32(c / c2); 8-bit code = nearest entry of
    the unsigned linear grid L8[q] = fl32(q / 255), ties to the lower code.
  * Dequantisation: c' = fl32(L8[q] * c2), w = fl32(Q[code] * c'), each a
    single IEEE fp32 multiply; an optional bf16 output is RNE of that fp32.

All arithmetic that decides an integer code is done in IEEE fp32 (numpy
float32 division), the precision of the block constants on the pages; the
comparisons against fp64 mid-points are exact because numpy widens float32
to float64 exactly.
"""

from fractions import Fraction
from statistics import NormalDist

import numpy as np

BLOCKSIZE = 64
GROUP = 256

# Upper end of the truncated normal: 1 - (1/32 + 1/30)/2 = 929/960.  NOT on
# the pages (they only say "truncated normal", [rkmt] §2.2.1); this value is
# the reading taken for the truncation point.
P_MAX = Fraction(1) - (Fraction(1, 32) + Fraction(1, 30)) / 2

ZERO_CODE = 7


def nf4_codebook_f64():
    """The 16 NF4 code points in fp64, ascending, spanning [-1, 1].

    [kwkr] §2.2: the code points are standard-normal quantiles, dense in the
    middle and sparse in the tails.  [rkmt] §2.2.1: quantiles of a truncated
    normal that cut the area under the density into equal parts.  [czcl]
    §2.1: an exact zero is kept.  Construction (reading): equal probability
    steps from 1/2 up to P_MAX on the positive side (8 steps) and on the
    negative side (7 steps), plus 0, divided by the quantile at P_MAX.
    The probabilities are formed exactly (Fractions) and rounded once.
    """
    inv_cdf = NormalDist(0.0, 1.0).inv_cdf
    half = Fraction(1, 2)
    pos = [inv_cdf(float(half + (P_MAX - half) * j / 8)) for j in range(1, 9)]
    neg = [-inv_cdf(float(half + (P_MAX - half) * j / 7)) for j in range(1, 8)]
    top = inv_cdf(float(P_MAX))
    q = np.array(sorted(neg + [0.0] + pos), dtype=np.float64)
    return q / top


def nf4_codebook():
    """The table the kernels use: the fp64 code points rounded to fp32 (RNE).

    [rkmt] §2.2.1 calls the looked-up value a 16-bit float; the compute type
    on the pages is bf16 ([rkmt] §3.2), so the table is kept in fp32 and the
    rounding to bf16 happens only where a bf16 operand is needed (reading).
    """
    return nf4_codebook_f64().astype(np.float32)


def nf4_midpoints():
    """fp64 mid-points between adjacent fp32 code points (exact in fp64)."""
    q = nf4_codebook().astype(np.float64)
    return (q[:-1] + q[1:]) / 2.0


def _as_f32_flat(w):
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).ravel()
    if not np.all(np.isfinite(w)):
        raise ValueError("oracle: inputs must be finite")
    return w


def quantize_nf4(w, blocksize=BLOCKSIZE):
    """Blockwise absmax NF4 quantisation.  Returns (packed uint8, absmax fp32).

    [rkmt] §2.2.2: each block of (for example) 64 weights gets one fp32
    quantisation constant; [kwkr] §3.1: block size 64.  [czcl] §2.1: each
    block is normalised on its own.  [rkmt] §2.2.1: every normalised weight
    maps to the nearest NF4 code point and only the 4-bit index is stored.
    The last block may be shorter (reading); ``w`` must have an even number
    of elements so the codes pack into whole bytes.
    """
    w = _as_f32_flat(w)
    n = w.size
    if n % 2:
        raise ValueError("oracle: numel must be even")
    nb = -(-n // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, blocksize)

    absmax = np.max(np.abs(blocks), axis=1)  # exact in fp32
    denom = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    v = blocks / denom[:, None]  # IEEE fp32 division, elementwise

    mids = nf4_midpoints()
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:  # nearest code, ties to the lower index
        codes += (v > m).astype(np.uint8)
    codes[absmax == 0] = ZERO_CODE  # an all-zero block stores exact zeros

    flat = codes.ravel()[:n]
    packed = ((flat[0::2] << 4) | flat[1::2]).astype(np.uint8)
    return packed, absmax.astype(np.float32)


def unpack_codes(packed, numel=None):
    """Inverse of the packing: even element from the high nibble."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    codes = np.empty(packed.size * 2, dtype=np.uint8)
    codes[0::2] = packed >> 4
    codes[1::2] = packed & 0x0F
    return codes if numel is None else codes[:numel]


def dq_levels():
    """The 256 level-2 code values fl32(q / 255), q = 0..255 (reading).

    [rkmt] §2.2.2 stores each block constant as an 8-bit integer plus an
    fp32 constant; the constants are non-negative, so the unsigned grid
    [0, 1] uses all 256 codes.
    """
    return np.arange(256, dtype=np.float32) / np.float32(255.0)


def double_quantize(absmax, group=GROUP):
    """Second quantisation of the fp32 block constants to 8 bits.

    [rkmt] §2.2.2 and [kwkr] §3.1: the quantisation constants are themselves
    quantised to 8 bits, with fp32 constants for the second level; [tgd] §2:
    this saves about 0.37 bit per parameter.  One fp32 constant per group of
    256 block constants (reading), the absmax of the group.
    Returns (q8 uint8[nblocks], c2 fp32[ceil(nblocks/group)]).
    """
    c = np.ascontiguousarray(np.asarray(absmax, dtype=np.float32)).ravel()
    if not np.all(np.isfinite(c)) or np.any(c < 0):
        raise ValueError("oracle: block constants must be finite and >= 0")
    nb = c.size
    ng = -(-nb // group)
    padded = np.zeros(ng * group, dtype=np.float32)
    padded[:nb] = c
    groups = padded.reshape(ng, group)

    c2 = np.max(groups, axis=1)
    denom = np.where(c2 > 0, c2, np.float32(1.0)).astype(np.float32)
    v = groups / denom[:, None]  # IEEE fp32 division

    lv = dq_levels().astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0
    q = np.zeros(groups.shape, dtype=np.int32)
    for m in mids:  # nearest level, ties to the lower code
        q += (v > m)
    return q.ravel()[:nb].astype(np.uint8), c2.astype(np.float32)


def dequant_scales(q8, c2, group=GROUP):
    """Recover the block constants: c' = fl32(L8[q] * c2[group of block])."""
    q8 = np.asarray(q8, dtype=np.uint8).ravel()
    c2 = np.asarray(c2, dtype=np.float32).ravel()
    gidx = np.arange(q8.size) // group
    return (dq_levels()[q8] * c2[gidx]).astype(np.float32)


def dequantize(packed, scales, numel, blocksize=BLOCKSIZE):
    """w = fl32(Q[code] * c') for every element.

    [rkmt] §2.2.1: dequantisation looks the stored 4-bit index up in the
    table; [kwkr] §2.3: the 4-bit weight is expanded to 16-bit only for the
    matrix product and never written back.  ``scales`` are the per-block
    constants (the fp32 absmax, or the double-dequantised c').
    """
    codes = unpack_codes(packed, numel)
    scales = np.asarray(scales, dtype=np.float32).ravel()
    q = nf4_codebook()
    return (q[codes] * scales[np.arange(numel) // blocksize]).astype(np.float32)


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16.

    Finite inputs only (the oracle asserts finiteness upstream).
    """
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f64_to_bf16_bits(x):
    """Round fp64 straight to bf16 (nearest, ties to even); returns uint16.

    x = m 2^e with 0.5 <= |m| < 1 has a bf16 spacing of 2^(e - 8) (8
    significant bits; never below the subnormal step 2^-133), so
    rint(x / spacing) * spacing is the rounding, exact in fp64, and the
    result is exactly representable in fp32.  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle: finite values only")
    _, e = np.frexp(x)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    y = np.rint(x / step) * step
    return (np.ascontiguousarray(y.astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
