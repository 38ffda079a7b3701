"""OCP OFP8 E5M2 codec.  Test infrastructure: see the package docstring.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2, quantizes activations to E5M2 (5
exponent bits, 2 mantissa bits: more range, less precision) while weights stay E4M3; page
"Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈" does not split the
formats.  This module is the OCP "OFP8" E5M2 variant (IEEE-like: bias 15, infinities and
NaNs in the top exponent), used by the E5M2-activation variant of the linear.

Byte layout ``s eeeee mm``:

* ``e == 0``              -> (-1)^s * m * 2^-16                (subnormals, +/-0 at m == 0)
* ``1 <= e <= 30``        -> (-1)^s * (4 + m) * 2^(e - 17)     (normals; largest 57344)
* ``e == 31, m == 0``     -> +/-infinity (0x7C, 0xFC)
* ``e == 31, m != 0``     -> NaN (0x7D-0x7F, 0xFD-0xFF)

Encoding (``encode``) is the saturating cast the quantizer uses, as for E4M3: NaN stays
NaN, magnitudes at or above 57344 (infinities included) become +/-57344 (0x7B / 0xFB),
everything else rounds to the nearest representable magnitude with ties to even, and the
sign is kept (-0 and negative underflow give 0x80).
"""

import numpy as np

MAX_FINITE = 57344.0
MIN_NORMAL = 2.0 ** -14
MIN_SUBNORMAL = 2.0 ** -16
BIAS = 15
MAX_CODE = 0x7B


def decode(codes):
    """E5M2 bytes -> float64 values (+/-inf and NaN in the top exponent), elementwise."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c >> 7) == 1
    e = (c >> 2) & 0x1F
    m = c & 0x3
    subnormal = m * MIN_SUBNORMAL
    normal = (4 + m) * np.exp2((e - 17).astype(np.float64))
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(neg, -mag, mag)


def encode(values):
    """float64 values -> E5M2 bytes: saturate to +/-57344, round to nearest even, keep sign.

    As in ``oracle.e4m3.encode``, powers of two scale exactly in float64 and ``np.rint``
    rounds half to even, so every step is exact.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)

    is_nan = np.isnan(a)
    is_sat = ~is_nan & (a >= MAX_FINITE)
    is_sub = ~is_nan & ~is_sat & (a < MIN_NORMAL)
    is_nrm = ~is_nan & ~is_sat & ~is_sub

    # Below the smallest normal the spacing is 2^-16; 4 units is the smallest normal, whose
    # byte is also 4 (e = 1, m = 0), so a carry needs no special case.
    code[is_sub] = np.rint(a[is_sub] / MIN_SUBNORMAL).astype(np.int64)

    # Normals: E = floor(log2 a), spacing 2^(E-2), significand n = a / spacing in [4, 8];
    # rounding up to 8 carries into the next binade.
    an = a[is_nrm]
    _, fexp = np.frexp(an)
    E = fexp.astype(np.int64) - 1
    n = np.rint(an / np.exp2((E - 2).astype(np.float64))).astype(np.int64)
    carry = n == 8
    E = np.where(carry, E + 1, E)
    n = np.where(carry, 4, n)
    code[is_nrm] = ((E + BIAS) << 2) | (n - 4)

    code[is_sat] = MAX_CODE
    code[is_nan] = 0x7F
    return (code | (neg << 7)).astype(np.uint8)


def table():
    """The 256 decoded values, indexed by byte."""
    return decode(np.arange(256, dtype=np.uint8))
