"""GPU row quantizer vs the oracle: bytes and scales bit-exact.

Covers the exhaustive FP16 sweep at unit scale, every FP16 amax, config-shaped rows at
every register-tiling width (and the wide-row loop path), launches whose workgroups walk
several row groups, zero and signed-zero rows,
saturation extremes, the SiLU*up prologue, the weight entry point over [B, N, K], and
determinism.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, quant
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu

ALL_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]
POS_FP16 = np.unique(FINITE_FP16[FINITE_FP16 > 0])


def _gpu_quant(x16):
    rq = require_gpu()
    x = dev(x16)
    q, s = rq.quant_weights(x)
    return host(q), host(s)


def _assert_exact(x16):
    q, s = _gpu_quant(x16)
    qr, sr = quant.quantize_rows(x16)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), "scale mismatch"
    bad = np.argwhere(q != qr)
    assert bad.size == 0, "byte mismatch at %s: gpu %s oracle %s x %s" % (
        bad[:5].tolist(), q[tuple(bad[0])], qr[tuple(bad[0])], x16[tuple(bad[0])])


def test_exhaustive_fp16_unit_scale():
    case("quant: all FP16 |v| <= 448 at s = 1")
    v = FINITE_FP16[np.abs(FINITE_FP16.astype(np.float64)) <= 448.0]
    per_row = 511
    pad = (-v.size) % per_row
    v = np.concatenate([v, np.zeros(pad, np.float16)]).reshape(-1, per_row)
    rows = np.concatenate([np.full((v.shape[0], 1), 448.0, np.float16), v], axis=1)
    _assert_exact(rows)


def test_every_fp16_amax():
    case("quant: every positive FP16 amax, K = 16")
    rng = np.random.default_rng(0)
    a = POS_FP16
    frac = rng.random((a.size, 15))
    sign = np.where(rng.random((a.size, 15)) < 0.5, -1.0, 1.0)
    x = (sign * frac * a.astype(np.float64)[:, None]).astype(np.float16)
    rows = np.concatenate([a[:, None], x], axis=1)
    rows[::2, 0] = -rows[::2, 0]
    _assert_exact(rows)


def test_amax_sweep_wide_rows():
    case("quant: amax sweep, K = 2048")
    rng = np.random.default_rng(1)
    a = POS_FP16[::8].astype(np.float64)
    sign = np.where(rng.random((a.size, 2047)) < 0.5, -1.0, 1.0)
    mag = rng.random((a.size, 2047)) ** 4          # many small and subnormal quotients
    x = (sign * mag * a[:, None]).astype(np.float16)
    rows = np.concatenate([a[:, None].astype(np.float16), x], axis=1)
    _assert_exact(rows)


@pytest.mark.parametrize("k", [16, 48, 512, 528, 1024, 2048, 4096, 8192, 8208, 16384])
@pytest.mark.parametrize("rows", [1, 5, 258])
def test_config_shaped_rows(k, rows):
    case("quant: rows=%d k=%d" % (rows, k))
    rng = np.random.default_rng(k * 1000 + rows)
    recipe = [workloads.acts_outliers, workloads.acts_channel_lognormal, workloads.acts_student_t][k % 3]
    x = recipe(rng, rows, k)
    _assert_exact(x)


@pytest.mark.parametrize("rows,k", [(10241, 2048), (20483, 512), (5121, 8192)])
def test_rows_walked_by_resident_workgroups(rows, k):
    # 2.5x as many row groups (4, 2 or 1 rows each) as a device of 256 CUs keeps resident:
    # the prefetching launch walks several groups per workgroup, and the first two shapes end
    # on a partly filled group
    case("quant: prefetching walk rows=%d k=%d" % (rows, k))
    rng = np.random.default_rng(rows + k)
    x = workloads.acts_student_t(rng, rows, k)
    _assert_exact(x)


def test_zero_signed_zero_and_extreme_rows():
    case("quant: special rows")
    x = np.zeros((6, 64), np.float16)
    x[1, ::3] = np.float16(-0.0)
    x[2, 5] = np.float16(2.0 ** -24)
    x[3, :] = np.float16(-65504.0)
    x[4, ::2] = np.float16(65504.0)
    x[4, 1::2] = np.float16(2.0 ** -24)
    x[5, :] = np.float16(-(2.0 ** -24))
    _assert_exact(x)
    q, _ = _gpu_quant(x)
    assert np.all(q[0] == 0) and np.all(q[1, ::3] == 0x80)


@pytest.mark.parametrize("k,rows", [(16, 3), (512, 65), (2048, 130), (4096, 33), (8192, 17), (8208, 5)])
def test_silu_mul_rows(k, rows):
    rq = require_gpu()
    case("quant: silu rows=%d k=%d" % (rows, k))
    rng = np.random.default_rng(k + rows)
    gu = (rng.standard_normal((rows, 2 * k)) * 3).astype(np.float16)
    gu[0, :4] = np.float16([0.0, -0.0, -60.0, 12.0])
    n = 16
    w_q = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    w_s = torch.ones((n,), dtype=torch.float32, device="cuda")
    _, dbg = rq.linear(dev(gu), w_q, w_s, act="silu_mul", debug=True)
    h = host(dbg["h"])
    h_ref = ffn.silu_mul(gu, k)
    d = ulp_diff16(h, h_ref)
    assert d.max() <= 1, "h off by %d ulp" % d.max()
    qr, sr = quant.quantize_rows(h)
    assert np.array_equal(host(dbg["a_scale"]).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(dbg["a_q"]), qr)


def test_weights_batched_matches_rows():
    rq = require_gpu()
    case("quant: weights [3, 80, 272]")
    rng = np.random.default_rng(2)
    w = workloads.weights(rng, (3, 80, 272))
    q, s = rq.quant_weights(dev(w))
    q, s = host(q), host(s)
    qr, sr = quant.quantize_rows(w.reshape(-1, 272))
    assert np.array_equal(q.reshape(-1, 272), qr)
    assert np.array_equal(s.reshape(-1).view(np.uint32), sr.view(np.uint32))


def test_full_size_activation_rows_and_determinism():
    rq = require_gpu()
    case("quant: 16384 x 2048 activation rows, twice")
    data = workloads.make(4, t=16384, k=2048, f=16, e=4)
    x = dev(data["x"])
    q1, s1 = rq.quant_weights(x)
    q2, s2 = rq.quant_weights(x)
    q1, s1, q2, s2 = host(q1), host(s1), host(q2), host(s2)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    qr, sr = quant.quantize_rows(data["x"])
    assert np.array_equal(s1.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q1, qr)
