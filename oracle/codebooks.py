"""Codebook variants of the 4-bit storage: the FP4 weight type, an FP8 level-2
code for the block constants, mean-centred double quantisation with a signed
8-bit code, and the uniform INT4 strawman; fp32 where a code is decided, fp64
elsewhere.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[kwkr] §4 and §4.1 offer "fp4" as the alternative quantisation type and
advise against it: it is made for floating-point-shaped distributions and
serves normally distributed weights worse than NF4.  The pages give no FP4
format.  Reading: the 4-bit float with one sign, two exponent and one
mantissa bit (E2M1), whose magnitudes are 0, 1/2, 1, 3/2, 2, 3, 4 and 6,
divided by 6 so a block's absmax maps to the largest code, exactly as NF4's
table spans [-1, 1].  Its 15 distinct values become a 16-entry ascending
table by entering 0 twice (indices 7 and 8; E2M1's -0 is not kept), so the
same nearest-code rule and packing as NF4 apply: code = number of fp64
mid-points strictly below fl32(w / c).

[kwkr] §3.1 compresses the fp32 block constants to "fp8".  Reading: the
ratio v = fl32(c / c2) in [0, 1] (c2 the group absmax, as for the 8-bit
integer code) is stored as an FP8 E4M3 number (4 exponent bits with bias 7,
3 mantissa bits, subnormals below 2^-6), rounded to nearest with ties to
the even code; the level value is that number itself, exact in fp32, and
c' = fl32(value * c2).  Every E4M3 number in [0, 1] has a code below 0x39.

Mean-centred double quantisation.  [rkmt] §2.2.2 and [kwkr] §3.1 quantise
the block constants a second time, to 8 bits; the pages stop there.  The
QLoRA publication they summarise also subtracts the mean of the constants
first, so that a symmetric signed code serves them.  Reading, step by step:
  1. offset mu = fl32(S / n), S the fp64 sum of the n constants taken by
     adjacent pairs (the constants, zero-padded to a power of two, are added
     0+1, 2+3, ... and the partial sums again, level by level), so the sum
     has one fixed order;
  2. centred constants d = fl32(c - mu);
  3. per group of 256, c2 = max |d|;
  4. t = fl32(d / c2) (t = 0 when c2 = 0) takes the nearest level of the
     signed grid fl32(k / 127), k = -127..127, ties toward k = 0; the code is
     k as a two's-complement byte;
  5. c' = fl32(fl32(fl32(k / 127) * c2) + mu).
Step 5 may give a slightly negative c' for a constant near 0 (the error is
at most half a level step of its group); that block's dequantised weights
then change sign, with magnitudes at that error's size.

[czcl] §2.1 shows a blockwise uniform 4-bit scheme as the contrast to NF4:
a symmetric grid of 15 evenly spaced levels whose outermost ones sit at
plus and minus the block's absmax.  It is not a storage format of the path;
it is kept as the strawman of the error study.
"""

from fractions import Fraction

import numpy as np

from . import nf4

_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _nearest_f32(fr):
    """The fp32 nearest to the rational fr, ties to the even significand."""
    f = np.float32(float(fr))
    cands = (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf)))
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.asarray(c).view(np.uint32)) & 1))
    return np.float32(best)


def fp4_codebook():
    """The 16 ascending FP4 code values (E2M1 / 6, zero entered twice), fp32."""
    mag = [Fraction(m) / 6 for m in _E2M1]
    vals = [-v for v in reversed(mag[1:])] + [Fraction(0), Fraction(0)] + mag[1:]
    return np.array([_nearest_f32(v) for v in vals], dtype=np.float32)


def codebook(kind):
    """'nf4' or 'fp4'."""
    if kind == "nf4":
        return nf4.nf4_codebook()
    if kind == "fp4":
        return fp4_codebook()
    raise ValueError(f"oracle: unknown codebook {kind!r}")


def quantize_4bit(w, kind, blocksize=nf4.BLOCKSIZE):
    """Blockwise absmax quantisation to the nearest entry of a 16-value table.

    The same steps as NF4 ([rkmt] §2.2.1-2.2.2): per block of 64 the fp32
    absmax c, v = fl32(w / c), code = number of fp64 mid-points of the table
    strictly below v, two codes per byte with the even element high.  An
    all-zero block takes the code of v = 0 (index 7 in both tables).
    """
    q = codebook(kind).astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2.0
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).ravel()
    if not np.all(np.isfinite(w)):
        raise ValueError("oracle: inputs must be finite")
    n = w.size
    if n % 2:
        raise ValueError("oracle: numel must be even")
    nb = -(-n // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, blocksize)
    absmax = np.max(np.abs(blocks), axis=1)
    denom = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    v = blocks / denom[:, None]
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:
        codes += (v > m).astype(np.uint8)
    codes[absmax == 0] = int(np.sum(mids < 0.0))
    flat = codes.ravel()[:n]
    packed = ((flat[0::2] << 4) | flat[1::2]).astype(np.uint8)
    return packed, absmax.astype(np.float32)


def dequantize_4bit(packed, scales, numel, kind, blocksize=nf4.BLOCKSIZE):
    """w = fl32(Q[code] * c') with the table of ``kind``."""
    codes = nf4.unpack_codes(packed, numel)
    scales = np.asarray(scales, dtype=np.float32).ravel()
    return (codebook(kind)[codes] * scales[np.arange(numel) // blocksize]).astype(np.float32)


def e4m3_values():
    """Value of every non-negative finite E4M3 code 0x00..0x7E (fp64, exact)."""
    out = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        out[code] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(v):
    """Nearest E4M3 code of each v in [0, 448], ties to the even code."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(v < 0) or np.any(v > 448.0):
        raise ValueError("oracle: e4m3_encode takes finite values in [0, 448]")
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in fp64
    code = np.searchsorted(mids, v, side="left")  # number of mid-points < v
    tie = (code < 126) & (v == mids[np.minimum(code, 125)])
    # at a tie v equals mids[code], between codes code and code + 1: take the even one
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    return code.astype(np.uint8)


def double_quantize_fp8(absmax, group=nf4.GROUP):
    """Level-2 code of the block constants as E4M3 numbers of fl32(c / c2)."""
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
    q = e4m3_encode(v.astype(np.float64))
    return q.ravel()[:nb], c2.astype(np.float32)


def dequant_scales_fp8(q8, c2, group=nf4.GROUP):
    """c' = fl32(E4M3 value of q * c2)."""
    q8 = np.asarray(q8, dtype=np.uint8).ravel()
    c2 = np.asarray(c2, dtype=np.float32).ravel()
    lv = e4m3_values().astype(np.float32)
    return (lv[q8] * c2[np.arange(q8.size) // group]).astype(np.float32)


def tree_sum_f64(values):
    """fp64 sum of the values by adjacent pairs: zero-padded to a power of two,
    then a[0::2] + a[1::2] level by level until one value is left."""
    a = np.asarray(values, dtype=np.float64).ravel()
    if a.size == 0:
        return 0.0
    n = 1
    while n < a.size:
        n *= 2
    a = np.concatenate([a, np.zeros(n - a.size)])
    while a.size > 1:
        a = a[0::2] + a[1::2]
    return float(a[0])


def centred_offset(absmax):
    """Step 1: mu = fl32(tree_sum_f64(c) / n), the offset subtracted from the
    block constants."""
    c = np.asarray(absmax, dtype=np.float32).ravel()
    if c.size == 0:
        return np.float32(0.0)
    return np.float32(tree_sum_f64(c) / float(c.size))


def s8_levels():
    """Level of every code byte: fl32(k / 127) for k the byte read as a
    two's-complement integer (byte 0x80, k = -128, is never produced)."""
    k = np.arange(256, dtype=np.int64)
    k = np.where(k >= 128, k - 256, k)
    return np.array([_nearest_f32(Fraction(int(v), 127)) for v in k], dtype=np.float32)


def s8_encode(t):
    """Step 4: code byte of each fp32 t in [-1, 1], nearest level of the grid
    fl32(k / 127), ties toward k = 0."""
    t = np.asarray(t, dtype=np.float32)
    lv = np.array([_nearest_f32(Fraction(j, 127)) for j in range(128)], dtype=np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0  # exact in fp64
    a = np.abs(t.astype(np.float64))
    j = np.searchsorted(mids, a, side="left")  # mid-points strictly below |t|
    k = np.where(t < 0, -j, j)
    return (k & 0xFF).astype(np.uint8)


def double_quantize_centred(absmax, group=nf4.GROUP):
    """Steps 1-4.  Returns (code bytes uint8[n], c2 fp32[ceil(n / group)], mu fp32)."""
    c = np.ascontiguousarray(np.asarray(absmax, dtype=np.float32)).ravel()
    if not np.all(np.isfinite(c)) or np.any(c < 0):
        raise ValueError("oracle: block constants must be finite and >= 0")
    mu = centred_offset(c)
    nb = c.size
    ng = -(-nb // group)
    d = np.zeros(ng * group, dtype=np.float32)
    d[:nb] = c - mu  # IEEE fp32 subtraction
    groups = d.reshape(ng, group)
    c2 = np.max(np.abs(groups), axis=1)
    denom = np.where(c2 > 0, c2, np.float32(1.0)).astype(np.float32)
    t = groups / denom[:, None]  # IEEE fp32 division; 0 / 1 = 0 for an all-zero group
    return s8_encode(t).ravel()[:nb], c2.astype(np.float32), mu


def dequant_scales_centred(q8, c2, mu, group=nf4.GROUP):
    """Step 5: c' = fl32(fl32(level of q * c2) + mu)."""
    q8 = np.asarray(q8, dtype=np.uint8).ravel()
    c2 = np.asarray(c2, dtype=np.float32).ravel()
    prod = (s8_levels()[q8] * c2[np.arange(q8.size) // group]).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


def int4_uniform_levels(absmax):
    """The 15 levels j * absmax / 7, j = -7..7, of one block (fp64)."""
    step = float(absmax) / 7.0
    return np.arange(-7, 8, dtype=np.float64) * step


def int4_uniform_roundtrip(w, blocksize=nf4.BLOCKSIZE):
    """Uniform symmetric 4-bit strawman ([czcl] §2.1), fp64.

    Each block of ``blocksize`` values is replaced by its nearest level of
    int4_uniform_levels(absmax of the block).  A value exactly half-way
    between two levels takes the one with the even index j (the half-to-even
    rounding of the page's framework).  An all-zero block stays zero.
    """
    w = np.asarray(w, dtype=np.float64).ravel()
    out = np.empty_like(w)
    for b0 in range(0, w.size, blocksize):
        blk = w[b0:b0 + blocksize]
        c = float(np.max(np.abs(blk)))
        if c == 0.0:
            out[b0:b0 + blocksize] = 0.0
            continue
        lv = int4_uniform_levels(c)
        dist = np.abs(blk[:, None] - lv[None, :])        # [values, 15 levels]
        best = dist.min(axis=1, keepdims=True)
        ties = dist == best
        # of the nearest levels (one, or two at a half-way point) keep the one
        # with the even index j = level position - 7
        even = (np.arange(15) - 7) % 2 == 0
        pick = np.where((ties & even[None, :]).any(axis=1),
                        np.argmax(ties & even[None, :], axis=1), np.argmax(ties, axis=1))
        out[b0:b0 + blocksize] = lv[pick]
    return out


def relative_mse(w, w_hat):
    """sum (w - w_hat)^2 / sum w^2, fp64."""
    w = np.asarray(w, dtype=np.float64).ravel()
    d = w - np.asarray(w_hat, dtype=np.float64).ravel()
    return float(np.sum(d * d) / np.sum(w * w))
