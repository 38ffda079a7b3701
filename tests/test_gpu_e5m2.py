"""GPU E5M2 activations x E4M3 weights vs the oracle.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2: activations quantized to E5M2,
weights to E4M3.  The quantized activation bytes and scales (the GEMM's operand, from the
debug outputs) must equal the oracle's E5M2 row quantizer bit for bit; FP16 outputs must
lie within the linear tolerance of the oracle's exact E5M2 x E4M3 product.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, linear, moe, quant, wscale
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu

FINITE_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE_FP16 = FINITE_FP16[np.isfinite(FINITE_FP16)]


def _quantized(rq, x16, k=None):
    """Run an E5M2 linear on x16 and return its quantized operand (bytes, scales)."""
    k = x16.shape[1] if k is None else k
    w_q = torch.zeros((16, k), dtype=torch.uint8, device="cuda")
    _, dbg = rq.linear(dev(x16), w_q, torch.ones(16, device="cuda"), debug=True, afmt="e5m2")
    return host(dbg["a_q"]), host(dbg["a_scale"])


def test_exhaustive_fp16_cast_at_unit_scale():
    """Every FP16 value within +/-57344 in a row whose maximum is 57344: s = 1 and the
    quotient is exact, so the bytes are the hardware cast itself against the OCP E5M2 one."""
    rq = require_gpu()
    case("e5m2 exhaustive FP16 cast")
    v = FINITE_FP16[np.abs(FINITE_FP16.astype(np.float64)) <= 57344.0]
    pad = (-v.size) % 15
    v = np.concatenate([v, np.zeros(pad, np.float16)]).reshape(-1, 15)
    rows = np.concatenate([np.full((v.shape[0], 1), 57344.0, np.float16), v], axis=1)
    q, s = _quantized(rq, rows)
    q_ref, s_ref = quant.quantize_rows(rows, "e5m2")
    assert np.all(s == np.float32(1.0))
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("m,k", [(1, 16), (7, 528), (300, 2048), (64, 8192), (5, 16384), (2000, 4096)])
def test_row_quantizer_bit_exact(m, k):
    """Every kernel variant: one or several wavefronts per row, and the two-pass loop past
    8192 values per row; Student-t rows stress the amax."""
    rq = require_gpu()
    case("e5m2 quantizer m=%d k=%d" % (m, k))
    rng = np.random.default_rng(m + k)
    x = workloads.acts_student_t(rng, m, k)
    x[0, :3] = np.float16(-0.0), np.float16(6e-8), np.float16(-65504.0)
    q, s = _quantized(rq, x)
    q_ref, s_ref = quant.quantize_rows(x, "e5m2")
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def _check(rq, x16, w16, tile=None, wscale_name="channel"):
    gran = {"channel": wscale.CHANNEL, "tensor": wscale.TENSOR, "block128": wscale.BLOCK128}[wscale_name]
    wq, ws = rq.quant_weights(dev(w16), wscale=wscale_name)
    y, dbg = rq.linear(dev(x16), wq, ws, debug=True, afmt="e5m2", wscale=wscale_name)
    xq, sx = quant.quantize_rows(x16, "e5m2")
    assert np.array_equal(host(dbg["a_q"]), xq)
    if gran == wscale.CHANNEL:
        ok, ratio, _ = linear.check(host(y), xq, sx, host(wq), host(ws), "e5m2")
    else:
        ok, ratio, _ = wscale.check(host(y), xq, sx, host(wq), host(ws), gran, "e5m2")
    assert ok, "max |d|/tol = %.3f" % ratio


@pytest.mark.parametrize("tile", [None, "256x256", "256x192", "256x128", "128x128", "64x128", "64x256"])
@pytest.mark.parametrize("m,n,k", [(130, 272, 528), (300, 384, 2048), (64, 128, 8192)])
def test_linear(monkeypatch, tile, m, n, k):
    rq = require_gpu()
    case("e5m2 linear tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(m * n + k)
    _check(rq, workloads.acts_channel_lognormal(rng, m, k), workloads.weights(rng, (n, k)))


@pytest.mark.parametrize("wscale_name", ["tensor", "block128"])
def test_linear_with_other_weight_scales(wscale_name):
    rq = require_gpu()
    case("e5m2 linear wscale=%s" % wscale_name)
    rng = np.random.default_rng(21)
    _check(rq, workloads.acts_student_t(rng, 200, 1024), workloads.weights(rng, (384, 1024)),
           wscale_name=wscale_name)


def test_gated_output_matches_the_unfused_path():
    rq = require_gpu()
    case("e5m2 gated linear")
    rng = np.random.default_rng(22)
    m, f, k = 130, 256, 512
    x = dev(workloads.acts_channel_lognormal(rng, m, k))
    order = ffn.gate_up_order(f)
    wq, ws = rq.quant_weights(dev(workloads.weights(rng, (2 * f, k))[order]))
    h = host(rq.linear(x, wq, ws, act="gate_silu", afmt="e5m2"))
    gu = host(rq.linear(x, wq, ws, afmt="e5m2"))
    gu_split = np.empty_like(gu)
    gu_split[:, order] = gu
    assert ulp_diff16(h, ffn.silu_mul(gu_split, f)).max() <= 1


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
def test_moe(monkeypatch, tile):
    """Tokens quantized once to E5M2 and scattered to their slots; grouped GEMM per expert."""
    rq = require_gpu()
    case("e5m2 moe tile=%s" % tile)
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    t, k, f, e = 300, 256, 96, 6
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids = d["ids"].astype(np.int32)
    wq, ws = rq.quant_weights(dev(d["w_gu"]))
    y, dbg = rq.moe_grouped_linear(dev(d["x"]), dev(ids), wq, ws, "tokens", "none", "permuted", debug=True,
                                   afmt="e5m2")
    xq, sx = quant.quantize_rows(d["x"], "e5m2")
    _, _, perm, _ = moe.plan(ids, e)
    assert np.array_equal(host(dbg["a_q"]), xq[perm // 2])
    ok, ratio = moe.grouped_linear_check(host(y), xq, sx, moe.IN_TOKENS, ids, host(wq), host(ws), a_fmt="e5m2")
    assert ok, ratio


def test_unknown_activation_format_is_rejected():
    rq = require_gpu()
    case("e5m2 argument errors")
    x = dev(np.zeros((4, 64), np.float16))
    with pytest.raises(rq.RqError):
        rq.linear(x, torch.zeros((16, 64), dtype=torch.uint8, device="cuda"), torch.ones(16, device="cuda"), afmt=7)


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
def test_moe_e5m2_with_block_scales(monkeypatch, tile):
    """Both variants at once: E5M2 token rows against 128x128-block-scaled E4M3 experts."""
    rq = require_gpu()
    case("e5m2 + block128 moe tile=%s" % tile)
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    t, k, f, e = 300, 256, 128, 6
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids = d["ids"].astype(np.int32)
    wq, ws = rq.quant_weights(dev(d["w_gu"]), wscale="block128")
    y, dbg = rq.moe_grouped_linear(dev(d["x"]), dev(ids), wq, ws, "tokens", "none", "permuted", debug=True,
                                   afmt="e5m2", wscale="block128")
    xq, sx = quant.quantize_rows(d["x"], "e5m2")
    ok, ratio = moe.grouped_linear_check(host(y), xq, sx, moe.IN_TOKENS, ids, host(wq), host(ws),
                                         gran=wscale.BLOCK128, a_fmt="e5m2")
    assert ok, ratio
