"""Row quantizer: one FP32 scale and E4M3 bytes per row.  Test infrastructure.

The same definition serves both granularities the pages name (page "Quantized
Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据): a weight
matrix [N out x K in] quantized per output channel is a row quantization of its N
rows, done once offline; an activation matrix [M tokens x K] quantized per token is a
row quantization of its M rows, done at run time.

Steps, after the per-token quantizer sketched on page "FP8量化在生成式推荐系统
OneRec-V2中的优化实践", §2.2 (scale from the row's absolute maximum with an epsilon
floor, then round and clamp), read for FP8 E4M3 with its +/-448 range (§1.2):

1. ``amax = max_i |x_i|`` over the FP16 row (exact).
2. ``s = fl32(max(amax, 2^-24) / 448)``: the FP32 dequantization scale, correctly
   rounded.  2^-24 is the smallest positive FP16, so only all-zero rows see the floor.
3. ``q_i = E4M3_SAT_RNE(fl32(x_i / s))``: the correctly rounded FP32 quotient, then the
   saturating round-to-nearest-even cast of ``oracle.e4m3.encode``.
4. Dequantization is ``decode(q_i) * s``.

Both FP32 roundings are computed as float64 quotients rounded to float32.  For one
division of FP32 operands that double rounding equals the single IEEE FP32 rounding,
because float64 carries more than 2*24+2 significand bits (Figueroa, "When is double
rounding innocuous?", 1995).
"""

import numpy as np

from . import e4m3, e5m2

EPS = 2.0 ** -24
QMAX = 448.0
# Target formats: codec and largest finite magnitude.  E5M2 (57344) serves the variant with
# E5M2 activations of page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2.
FORMATS = {"e4m3": (e4m3, QMAX), "e5m2": (e5m2, e5m2.MAX_FINITE)}


def row_scale(amax, qmax=QMAX):
    """FP32 scale per row from the rows' absolute maxima (float64 in, float32 out)."""
    amax = np.asarray(amax, dtype=np.float64)
    return (np.maximum(amax, EPS) / qmax).astype(np.float32)


def quantize_rows(x, fmt="e4m3"):
    """Quantize each row of a 2-D FP16 array to ``fmt`` ("e4m3", or "e5m2" with 57344 in
    place of 448).

    Returns ``(q, s)``: ``q`` uint8 bytes with the shape of ``x`` and ``s`` float32 scales,
    one per row.
    """
    codec, qmax = FORMATS[fmt]
    x16 = np.asarray(x)
    if x16.dtype != np.float16:
        raise TypeError("the quantizer takes FP16 rows")
    if x16.ndim != 2:
        raise ValueError("expected a 2-D array of rows")
    rows, k = x16.shape
    if rows == 0:
        return np.zeros((0, k), np.uint8), np.zeros((0,), np.float32)
    xd = x16.astype(np.float64)
    amax = np.max(np.abs(xd), axis=1) if k > 0 else np.zeros(rows)
    s = row_scale(amax, qmax)
    quotient = (xd / s.astype(np.float64)[:, None]).astype(np.float32)
    q = codec.encode(quotient.astype(np.float64))
    return q, s


def dequantize_rows(q, s, fmt="e4m3"):
    """float64 values ``decode(q) * s`` (row-wise scale)."""
    return FORMATS[fmt][0].decode(q) * np.asarray(s, dtype=np.float64)[:, None]
