"""Pins of the oracle's W8A8 linear: exact brute force, a textbook reduction, invariants.

The linear follows page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化
栈", section 关键证据 (FP8 products, FP32 accumulation, FP16 output) and page
"FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.3 / Fig. 2.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, linear, quant

FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _frac_decode(c):
    c = int(c)
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m) * (Fraction(2) ** (e - 10))


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 4, 32), (5, 9, 48)])
def test_gemm_exact_matches_fraction_brute_force(shape):
    m, n, k = shape
    rng = np.random.default_rng(sum(shape))
    xq = rng.choice(FINITE_CODES, size=(m, k))
    wq = rng.choice(FINITE_CODES, size=(n, k))
    xq[0, 0] = 0x7E
    wq[0, 0] = 0x7E       # a 448 * 448 product
    if k > 1:
        xq[-1, -1] = 0x01
        wq[-1, -1] = 0x81  # a subnormal * negative subnormal product
    acc = linear.gemm_exact(xq, wq)
    absacc = linear.gemm_abs_exact(xq, wq)
    for i in range(m):
        for j in range(n):
            exact = sum(_frac_decode(xq[i, t]) * _frac_decode(wq[j, t]) for t in range(k))
            exact_abs = sum(abs(_frac_decode(xq[i, t]) * _frac_decode(wq[j, t])) for t in range(k))
            assert Fraction(acc[i, j]) == exact
            assert Fraction(absacc[i, j]) == exact_abs


def test_exact_at_largest_k():
    # All products +448*448 over K = 8192: the sum 8192 * 200704 must be exact.
    xq = np.full((2, 8192), 0x7E, np.uint8)
    wq = np.full((3, 8192), 0x7E, np.uint8)
    wq[1] = 0xFE
    acc = linear.gemm_exact(xq, wq)
    assert np.all(acc[:, 0] == 8192 * 448.0 * 448.0)
    assert np.all(acc[:, 1] == -8192 * 448.0 * 448.0)


def test_dequantize_rounds_once_to_fp16():
    acc = np.array([[1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0 + 15.0, 2.0 ** -25]])
    y = linear.dequantize_fp16(acc, np.array([1.0], np.float32), np.ones(4, np.float32))
    # ties to even: 1 + 2^-11 -> 1, 1 + 3*2^-11 -> 1 + 2^-9; 65519 -> 65504; 2^-25 -> 0
    assert y[0].tolist() == [1.0, 1.0 + 2.0 ** -9, 65504.0, 0.0]


def test_power_of_two_scaled_inputs_reduce_to_plain_matmul():
    # Rows built from E4M3 values times 2^a_m that contain +/-448 * 2^a_m quantize with
    # s_x[m] = 2^a_m exactly and no rounding (same for weight rows with 2^b_n), so the
    # quantized linear must equal fl16 of the plain float64 matmul of the FP16 inputs.
    # Row-dependent exponents catch a swapped or mis-indexed scale; M != N != K catches
    # a transposed operand.
    rng = np.random.default_rng(21)
    m, n, k = 7, 5, 40
    a = rng.integers(-6, 3, size=m)
    b = rng.integers(-9, -3, size=n)
    xv = e4m3.decode(rng.choice(FINITE_CODES, size=(m, k)))
    wv = e4m3.decode(rng.choice(FINITE_CODES, size=(n, k)))
    xv[:, 3] = 448.0
    wv[:, 1] = -448.0
    x = (xv * np.exp2(a)[:, None]).astype(np.float16)
    w = (wv * np.exp2(b)[:, None]).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), xv * np.exp2(a)[:, None])
    xq, sx = quant.quantize_rows(x)
    wq, sw = quant.quantize_rows(w)
    assert np.array_equal(sx, np.exp2(a).astype(np.float32))
    assert np.array_equal(sw, np.exp2(b).astype(np.float32))
    y = linear.linear(xq, sx, wq, sw)
    ref = (x.astype(np.float64) @ w.astype(np.float64).T).astype(np.float16)
    assert np.array_equal(y, ref)


def test_merged_qkv_equals_three_linears():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 64)).astype(np.float16)
    wq_ = (rng.standard_normal((48, 64)) * 0.02).astype(np.float16)
    xq, sx = quant.quantize_rows(x)
    wq, sw = quant.quantize_rows(wq_)
    merged = linear.linear(xq, sx, wq, sw)
    parts = [linear.linear(xq, sx, *quant.quantize_rows(wq_[i:i + 16])) for i in (0, 16, 32)]
    assert np.array_equal(merged, np.concatenate(parts, axis=1))


def test_zero_row_gives_zero_output():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 32)).astype(np.float16)
    x[2] = 0
    w = rng.standard_normal((6, 32)).astype(np.float16)
    y = linear.linear(*quant.quantize_rows(x), *quant.quantize_rows(w))
    assert np.all(y[2] == 0)


def test_ulp16_closed_forms():
    v = np.array([0.0, 1.0, -1.0, 1.5, 2.0, 65504.0, 2.0 ** -14, 2.0 ** -15, 2.0 ** -24, 1000.0])
    assert linear.ulp16(v).tolist() == [2.0 ** -24, 2.0 ** -10, 2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 32.0,
                                        2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 0.5]


def test_check_accepts_reference_and_rejects_perturbed():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 128)).astype(np.float16)
    w = (rng.standard_normal((24, 128)) * 0.02).astype(np.float16)
    xq, sx = quant.quantize_rows(x)
    wq, sw = quant.quantize_rows(w)
    ok, ratio, yref = linear.check(linear.linear(xq, sx, wq, sw), xq, sx, wq, sw)
    assert ok and ratio == 0.0
    bad = yref.astype(np.float64)
    bad[3, 4] += 0.25 + abs(bad[3, 4])
    ok, ratio, _ = linear.check(bad, xq, sx, wq, sw)
    assert not ok and ratio > 1
