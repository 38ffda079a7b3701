"""W8A8 FP8 linear: exact FP8 dot products, dequantization, FP16 output.  Test infrastructure.

Follows page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈",
section 关键证据 (FP8 products accumulated in FP32, output cast back to FP16) and page
"FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.3 and Fig. 2 (FP8 multiply, FP32
accumulation, FP16 output; dynamic quantization before the GEMM, dequantization after).

Layout: activations ``x_q`` [M x K] (one row per token), weights ``w_q`` [N x K] (one row
per output channel, the nn.Linear layout), scales ``s_x`` [M] and ``s_w`` [N].  No bias:
the pages never mention one.

Exactness of the accumulation.  Every E4M3 value is an integer multiple of 2^-9 with
magnitude at most 448, so after multiplying by 2^9 the operands are integers below
2^17.8, each product is an integer below 2^35.6 and any partial sum over K <= 2^17
terms stays below 2^53.  A float64 matrix product of the integer-scaled operands is
therefore exact in every summation order, BLAS included.  The oracle's accumulator is
the exact real dot product; the "FP32 accumulation" of the pages is what the tolerance
below allows for.

With E5M2 activations (the variant of page "FP8量化在生成式推荐系统OneRec-V2中的优化实践",
§2.2) the activation operand is an integer multiple of 2^-16 below 2^15.8, so the integer
products reach 2^49.6 and sums over K <= 8192 reach 2^62.6: those are accumulated in int64,
exact below 2^63.

Output: ``y* = acc * s_x[m] * s_w[n]`` in float64, then one round-to-nearest-even to
FP16 (numpy's float64 -> float16 cast rounds directly, ties to even).

Tolerance for a GPU result ``y`` against ``y_ref = fl16(y*)``:

    |y - y_ref| <= 2 * ulp16(y_ref) + 1e-3 * s_x[m] * s_w[n] * sum_k |dec(x_q) * dec(w_q)|

with ``ulp16(v) = 2^(max(floor(log2|v|), -14) - 10)`` and ``ulp16(0) = 2^-24``.  The first
term covers the FP32 epilogue and the final FP16 rounding, the second any FP32
summation order of the K products.
"""

import numpy as np

from . import e4m3, e5m2

# E4M3 values are integer multiples of 2^-9, E5M2 values of 2^-16.
_UNITS = {"e4m3": (e4m3, 2.0 ** 9), "e5m2": (e5m2, 2.0 ** 16)}


def _int_operand(codes, fmt="e4m3"):
    codec, unit = _UNITS[fmt]
    vals = codec.decode(codes)
    if not np.isfinite(vals).all():
        raise ValueError("NaN or infinite %s code in a GEMM operand" % fmt)
    return vals * unit


def _exact_products(a, b, scale):
    """a @ b.T / scale for integer-valued float64 operands, exactly."""
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    bound = np.max(np.abs(a), initial=0.0) * np.max(np.abs(b), initial=0.0) * a.shape[1]
    if bound < 2.0 ** 53:
        return (a @ b.T) / scale                       # every partial sum is an exact float64
    if bound >= 2.0 ** 63:
        raise ValueError("K too large for exact accumulation")
    # E5M2 activations: integer products reach 2^49.6, so sum them in int64 (exact below 2^63)
    return (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64) / scale


def gemm_exact(x_q, w_q, a_fmt="e4m3"):
    """Exact ``acc[m, n] = sum_k dec(x_q[m, k]) * dec(w_q[n, k])`` as float64 (activations in
    ``a_fmt``, weights E4M3)."""
    return _exact_products(_int_operand(x_q, a_fmt), _int_operand(w_q), _UNITS[a_fmt][1] * 2.0 ** 9)


def gemm_abs_exact(x_q, w_q, a_fmt="e4m3"):
    """Exact ``sum_k |dec(x_q[m, k]) * dec(w_q[n, k])|`` as float64."""
    return _exact_products(np.abs(_int_operand(x_q, a_fmt)), np.abs(_int_operand(w_q)),
                           _UNITS[a_fmt][1] * 2.0 ** 9)


def dequantize_fp16(acc, s_x, s_w):
    """``fl16(acc * s_x[m] * s_w[n])`` with the products in float64."""
    sx = np.asarray(s_x, dtype=np.float64)[:, None]
    sw = np.asarray(s_w, dtype=np.float64)[None, :]
    return (acc * sx * sw).astype(np.float16)


def linear(x_q, s_x, w_q, s_w, a_fmt="e4m3"):
    """FP16 output of the quantized linear for quantized operands."""
    return dequantize_fp16(gemm_exact(x_q, w_q, a_fmt), s_x, s_w)


def ulp16(y):
    """FP16 unit in the last place of each value (2^-24 at zero and in the subnormals)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    out = np.full(a.shape, 2.0 ** -24)
    nz = a > 0
    _, fexp = np.frexp(a[nz])
    e = np.maximum(fexp.astype(np.int64) - 1, -14)
    out[nz] = np.exp2((e - 10).astype(np.float64))
    return out


def tolerance(y_ref, s_x, s_w, abs_acc):
    """Per-element bound on |y_gpu - y_ref| (see the module docstring)."""
    sx = np.asarray(s_x, dtype=np.float64)[:, None]
    sw = np.asarray(s_w, dtype=np.float64)[None, :]
    return 2.0 * ulp16(y_ref) + 1e-3 * sx * sw * abs_acc


def check(y_gpu, x_q, s_x, w_q, s_w, a_fmt="e4m3"):
    """Compare a GPU output with the oracle.  Returns ``(ok, worst |d|/tol, y_ref)``."""
    y_ref = linear(x_q, s_x, w_q, s_w, a_fmt)
    tol = tolerance(y_ref, s_x, s_w, gemm_abs_exact(x_q, w_q, a_fmt))
    d = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref.astype(np.float64))
    bad = ~(d <= tol)
    ratio = float(np.max(d / tol)) if d.size else 0.0
    return (not bad.any()), ratio, y_ref
