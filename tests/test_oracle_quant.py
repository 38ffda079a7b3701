"""Pins of the oracle's row quantizer (closed forms, invariants, special cases).

The quantizer follows the per-token recipe of page "FP8量化在生成式推荐系统OneRec-V2中
的优化实践", §2.2 (amax-derived scale with an epsilon floor, round, clamp), read for
E4M3 with the +/-448 range of §1.2; page "Quantized Inference for OneRec-V2：生成式推荐
开始直接吃 LLM 量化栈", section 关键证据, applies it per output channel to weights and
per token to activations.
"""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import e4m3, quant

ALL_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]
POS_FP16 = np.unique(FINITE_FP16[FINITE_FP16 > 0])


def test_scale_is_fp32_division():
    # fl32(amax / 448) computed as float64 then rounded must equal PyTorch's float32
    # division (IEEE, a single rounding) for every positive FP16 amax.
    ours = quant.row_scale(POS_FP16.astype(np.float64))
    ref = (torch.from_numpy(POS_FP16.astype(np.float32)) / torch.tensor(448.0, dtype=torch.float32)).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_quotient_is_fp32_division():
    rng = np.random.default_rng(3)
    x = rng.choice(FINITE_FP16, size=(64, 2048))
    q, s = quant.quantize_rows(x)
    quot_ref = (torch.from_numpy(x.astype(np.float32)) / torch.from_numpy(s)[:, None]).numpy()
    assert np.array_equal(q, torch.from_numpy(quot_ref).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_amax_maps_to_448_for_every_fp16_amax():
    rows = np.stack([POS_FP16, -POS_FP16, POS_FP16 * np.float16(0.5)], axis=1)
    q, s = quant.quantize_rows(rows)
    assert POS_FP16.size == 31743
    assert np.all(q[:, 0] == 0x7E)
    assert np.all(q[:, 1] == 0xFE)


def test_exhaustive_fp16_at_unit_scale():
    # Every row holds +448, so amax = 448, s = 1 exactly and the quotient is exact:
    # the quantizer reduces to the plain cast, checked against PyTorch's cast.
    v = FINITE_FP16[np.abs(FINITE_FP16.astype(np.float64)) <= 448.0]
    rows = np.stack([np.full(v.shape, 448.0, np.float16), v], axis=1)
    q, s = quant.quantize_rows(rows)
    assert np.all(s == np.float32(1.0))
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[:, 1], ref)


def test_zero_rows():
    x = np.zeros((3, 64), np.float16)
    x[1, ::2] = np.float16(-0.0)
    q, s = quant.quantize_rows(x)
    assert np.all(s == np.float32(2.0 ** -24 / 448.0))
    assert np.all(q[0] == 0x00)
    assert np.all(q[1, ::2] == 0x80) and np.all(q[1, 1::2] == 0x00)
    assert np.all(e4m3.decode(q) * s[:, None].astype(np.float64) == 0.0)


@pytest.mark.parametrize("j", list(range(-15, 8)))
def test_power_of_two_rows_are_exact(j):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes) * 2.0 ** j
    row = vals.astype(np.float16)
    assert np.array_equal(row.astype(np.float64), vals)  # representable in FP16
    q, s = quant.quantize_rows(row[None, :])
    assert s[0] == np.float32(2.0 ** j)
    assert np.array_equal(q[0], codes)


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((32, 256)) * 3).astype(np.float16)
    q, s = quant.quantize_rows(x)
    qn, sn = quant.quantize_rows(-x)
    assert np.array_equal(sn, s)
    assert np.array_equal(qn, q ^ 0x80)
    for j in (-3, 2, 5):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** j)
        qj, sj = quant.quantize_rows(xs)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s.astype(np.float64) * 2.0 ** j).astype(np.float32))


def test_saturation_and_no_nan():
    rng = np.random.default_rng(9)
    x = rng.choice(FINITE_FP16, size=(256, 512))
    x[:, 0] = np.float16(65504.0)
    x[:, 1] = np.float16(-65504.0)
    q, s = quant.quantize_rows(x)
    d = e4m3.decode(q)
    assert not np.isnan(d).any()
    assert np.abs(d).max() <= 448.0


def test_rows_are_independent():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((40, 96)) * np.exp2(rng.uniform(-8, 8, (40, 1)))).astype(np.float16)
    q, s = quant.quantize_rows(x)
    for i in (0, 17, 39):
        qi, si = quant.quantize_rows(x[i:i + 1])
        assert np.array_equal(qi[0], q[i]) and si[0] == s[i]


fp16_finite = st.integers(0, 65535).map(lambda b: np.array([b], np.uint16).view(np.float16)[0]).filter(
    lambda v: np.isfinite(v))


@settings(max_examples=300, deadline=None)
@given(st.lists(fp16_finite, min_size=1, max_size=64))
def test_error_bound_and_monotonicity(vals):
    x = np.array(vals, np.float16)[None, :]
    q, s = quant.quantize_rows(x)
    xd = x.astype(np.float64)[0]
    sd = float(s[0])
    y = e4m3.decode(q[0]) * sd
    r = np.abs(xd / sd)
    normal = r >= 2.0 ** -6
    err = np.abs(xd - y)
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -23) * np.abs(xd[normal]) * (1 + 1e-12))
    assert np.all(err[~normal] <= 2.0 ** -10 * sd + 2.0 ** -23 * np.abs(xd[~normal]) + 1e-300)
    order = np.argsort(xd, kind="stable")
    deq = e4m3.decode(q[0])[order]
    assert np.all(np.diff(deq) >= 0)


def test_empty_rows():
    q, s = quant.quantize_rows(np.zeros((0, 32), np.float16))
    assert q.shape == (0, 32) and s.shape == (0,)
