"""GPU weight scales per tensor and per 128 x 128 block vs the oracle (oracle.wscale).

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1 / §2.2: dense FFN weights with one
scale per tensor, MoE expert weights with one scale per 128 x 128 block.  Weight bytes and
scales must equal the oracle's bit for bit; FP16 outputs must lie within the block-wise
tolerance of ``oracle.wscale.check``, evaluated on the GPU's own quantized activations.
The weights are skewed per block (factors from 1/16 to 16 along K and 1/2 to 2 along N,
plus an all-zero block) so that consecutive K-block scales differ widely, and the zero
block exercises the floor scale.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, moe, quant, wscale
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu

GRAN = {"tensor": wscale.TENSOR, "block128": wscale.BLOCK128}


def _skewed(rng, n, k, zero_block=True):
    w = workloads.weights(rng, (n, k)).astype(np.float64)
    if n % 128 == 0 and k % 128 == 0:
        fk = rng.choice([1 / 16, 1 / 4, 1.0, 4.0, 16.0], size=k // 128)
        fn = rng.choice([0.5, 1.0, 2.0], size=n // 128)
        w *= np.repeat(fn, 128)[:, None] * np.repeat(fk, 128)[None, :]
        if zero_block and k >= 256:
            w[:128, 128:256] = 0.0
    return w.astype(np.float16)


def _oracle_quant(w16, gran):
    if w16.ndim == 2:
        return wscale.quantize(w16, GRAN[gran])
    qs = [wscale.quantize(m, GRAN[gran]) for m in w16]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs]).reshape(
        (w16.shape[0],) if gran == "tensor" else (w16.shape[0],) + qs[0][1].shape)


@pytest.mark.parametrize("gran,shape", [
    ("tensor", (96, 160)), ("tensor", (4, 48, 272)), ("tensor", (256, 384)), ("tensor", (2048, 4096)),
    ("block128", (128, 128)), ("block128", (256, 384)), ("block128", (3, 256, 512)), ("block128", (2048, 4096)),
])
def test_weight_quantization_bit_exact(gran, shape):
    rq = require_gpu()
    case("weight quant %s %r" % (gran, shape))
    rng = np.random.default_rng(sum(shape))
    if len(shape) == 2:
        w = _skewed(rng, *shape)
    else:
        w = np.stack([_skewed(rng, *shape[1:]) for _ in range(shape[0])])
    w[..., 0, 1] = np.float16(-0.0)
    w[..., 1, 2] = np.float16(3e-7)                      # an FP16 subnormal
    wq, ws = rq.quant_weights(dev(w), wscale=gran)
    q_ref, s_ref = _oracle_quant(w, gran)
    assert tuple(ws.shape) == s_ref.shape
    assert np.array_equal(host(wq), q_ref)
    assert np.array_equal(host(ws).view(np.uint32), s_ref.astype(np.float32).view(np.uint32))


def _check_linear(rq, x16, w16, gran, act="none"):
    wq, ws = rq.quant_weights(dev(w16), wscale=gran)
    y, dbg = rq.linear(dev(x16), wq, ws, act=act, debug=True, wscale=gran)
    xq_ref, sx_ref = quant.quantize_rows(x16)
    assert np.array_equal(host(dbg["a_q"]), xq_ref)
    ok, ratio, _ = wscale.check(host(y), xq_ref, sx_ref, host(wq), host(ws), GRAN[gran])
    assert ok, "max |d|/tol = %.3f" % ratio
    return ratio


@pytest.mark.parametrize("gran", ["tensor", "block128"])
@pytest.mark.parametrize("tile", [None, "256x256", "256x192", "256x128", "128x128", "64x128", "64x256"])
@pytest.mark.parametrize("m,n,k", [(130, 384, 512), (300, 256, 2048), (64, 128, 256)])
def test_linear(monkeypatch, gran, tile, m, n, k):
    """Short K (only the generic slab steps: each K block's rescale decided at run time) and
    K = 2048 (the steady steps, with the rescale compiled into every second slab)."""
    rq = require_gpu()
    case("linear wscale=%s tile=%s m=%d n=%d k=%d" % (gran, tile, m, n, k))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(m + n + k)
    _check_linear(rq, workloads.acts_channel_lognormal(rng, m, k), _skewed(rng, n, k), gran)


@pytest.mark.parametrize("grid", ["3", "8"])
@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x256"])
def test_block_linear_persistent_walk(monkeypatch, grid, tile):
    """Few workgroups walking many tiles: each tile restarts its scale row and its K blocks."""
    rq = require_gpu()
    case("block linear walk grid=%s tile=%s" % (grid, tile))
    monkeypatch.setenv("RQ_GEMM_TILE", tile)
    monkeypatch.setenv("RQ_GEMM_GRID", grid)
    rng = np.random.default_rng(7)
    _check_linear(rq, workloads.acts_student_t(rng, 300, 1024), _skewed(rng, 640, 1024), "block128")


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
def test_block_gated_output(monkeypatch, tile):
    """act='gate_silu' with block scales on interleaved gate/up rows: h is the SiLU*up that
    the quantizer's own transform makes of the plain block-scaled linear's FP16 outputs, bit
    for bit, and within 1 FP16 ulp of the oracle's SiLU of them; the plain linear itself is
    within the block tolerance."""
    rq = require_gpu()
    case("block gated tile=%s" % tile)
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(8)
    m, f, k = 130, 128, 512
    x16 = workloads.acts_channel_lognormal(rng, m, k)
    order = ffn.gate_up_order(f)
    w = _skewed(rng, 2 * f, k)[order]
    _check_linear(rq, x16, w, "block128")
    x = dev(x16)
    wq, ws = rq.quant_weights(dev(w), wscale="block128")
    h = host(rq.linear(x, wq, ws, act="gate_silu", wscale="block128"))
    gu = host(rq.linear(x, wq, ws, wscale="block128"))
    gu_split = np.empty_like(gu)
    gu_split[:, order] = gu                                   # back to [g (F) | u (F)]
    w_dn_q = torch.zeros((16, f), dtype=torch.uint8, device="cuda")
    _, dbg = rq.linear(dev(gu_split), w_dn_q, torch.ones(16, device="cuda"), act="silu_mul", debug=True)
    assert np.array_equal(h.view(np.uint16), host(dbg["h"]).view(np.uint16))
    assert ulp_diff16(h, ffn.silu_mul(gu_split, f)).max() <= 1


def _moe_block(rq, d, t, k, f, e, top_k, sample=None):
    """Block-scaled expert FFN: gate/up (TOKENS) then down (PERMUTED, SILU_MUL, COMBINED)."""
    ids = d["ids"].astype(np.int32)
    wgu_q, wgu_s = rq.quant_weights(dev(d["w_gu"]), wscale="block128")
    wdn_q, wdn_s = rq.quant_weights(dev(d["w_dn"]), wscale="block128")
    for ex in range(0, e, max(1, e // 4)):                     # weight bytes: a few experts
        q_ref, s_ref = wscale.quantize_blocks(d["w_gu"][ex])
        assert np.array_equal(host(wgu_q[ex]), q_ref) and np.array_equal(host(wgu_s[ex]), s_ref)
    x, ids_d, tw = dev(d["x"]), dev(ids), dev(d["topk_w"])
    gu, dbg1 = rq.moe_grouped_linear(x, ids_d, wgu_q, wgu_s, "tokens", "none", "permuted", debug=True,
                                     wscale="block128")
    gu_h, aq1, as1 = host(gu), host(dbg1["a_q"]), host(dbg1["a_scale"])
    counts, offsets, perm, pos = moe.plan(ids, e)
    xq, xs = quant.quantize_rows(d["x"])
    assert np.array_equal(aq1, xq[perm // top_k])
    rows = np.arange(t * top_k) if sample is None else np.asarray(sample)
    wgu_qh, wgu_sh = host(wgu_q), host(wgu_s)
    experts = np.searchsorted(offsets, rows, side="right") - 1
    for ex in np.unique(experts):
        r = rows[experts == ex]
        ok, ratio, _ = wscale.check(gu_h[r], aq1[r], as1[r], wgu_qh[ex], wgu_sh[ex], wscale.BLOCK128)
        assert ok, (int(ex), ratio)
    out, dbg2 = rq.moe_grouped_linear(gu, ids_d, wdn_q, wdn_s, "permuted", "silu_mul", "combined", topk_w=tw,
                                      debug=True, wscale="block128")
    y_perm = host(rq.moe_grouped_linear(gu, ids_d, wdn_q, wdn_s, "permuted", "silu_mul", "permuted",
                                        wscale="block128"))
    aq2, as2 = host(dbg2["a_q"]), host(dbg2["a_scale"])
    wdn_qh, wdn_sh = host(wdn_q), host(wdn_s)
    for ex in np.unique(experts):
        r = rows[experts == ex]
        ok, ratio, _ = wscale.check(y_perm[r], aq2[r], as2[r], wdn_qh[ex], wdn_sh[ex], wscale.BLOCK128)
        assert ok, (int(ex), ratio)
    if sample is None:
        assert ulp_diff16(host(out), moe.combine(y_perm, pos, d["topk_w"])).max() <= 1
        # the oracle's own per-expert check over every permuted row, from the token rows
        ok, ratio = moe.grouped_linear_check(gu_h, xq, xs, moe.IN_TOKENS, ids, wgu_qh, wgu_sh, gran=wscale.BLOCK128)
        assert ok, ratio


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
@pytest.mark.parametrize("t,k,f,e,top_k", [(300, 256, 128, 6, 2), (129, 512, 256, 8, 1)])
def test_moe_block_scales(monkeypatch, tile, t, k, f, e, top_k):
    rq = require_gpu()
    case("moe block tile=%s t=%d k=%d f=%d e=%d top_k=%d" % (tile, t, k, f, e, top_k))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    d = workloads.make(4, t=t, k=k, f=f, e=e, top_k=top_k)
    _moe_block(rq, d, t, k, f, e, top_k)


def test_tensor_scales_moe():
    """Per-tensor expert scales ([E]) through the grouped GEMM."""
    rq = require_gpu()
    case("moe tensor scales")
    d = workloads.make(4, t=200, k=256, f=96, e=5)
    ids = d["ids"].astype(np.int32)
    wq, ws = rq.quant_weights(dev(d["w_gu"]), wscale="tensor")
    assert tuple(ws.shape) == (5,)
    y, dbg = rq.moe_grouped_linear(dev(d["x"]), dev(ids), wq, ws, "tokens", "none", "permuted", debug=True,
                                   wscale="tensor")
    ok, ratio = moe.grouped_linear_check(host(y), host(dbg["a_q"]), host(dbg["a_scale"]), moe.IN_PERMUTED,
                                         ids, host(wq), host(ws).reshape(5, 1), gran=wscale.TENSOR)
    assert ok, ratio


def test_block_scales_need_128_multiples():
    rq = require_gpu()
    case("block alignment errors")
    w = dev(np.zeros((128, 192), np.float16))
    with pytest.raises(rq.RqError):
        rq.quant_weights(w, w_scale=torch.empty((1, 1), device="cuda"), wscale="block128")
    x = dev(np.zeros((4, 192), np.float16))
    with pytest.raises(rq.RqError):
        rq.linear(x, torch.zeros((128, 192), dtype=torch.uint8, device="cuda"),
                  torch.ones((1, 1), device="cuda"), wscale="block128")


@pytest.mark.slow
def test_moe_block_full_size_sampled():
    """The MoE workload (16384 tokens, top-2 of 32 Zipf-loaded experts, F = 4096) with block
    scales, on the first and last row of every expert and 64 random rows."""
    rq = require_gpu()
    case("workload 4 with 128x128 block scales")
    d = workloads.make(4)
    rng = np.random.default_rng(44)
    counts, offsets, _, _ = moe.plan(d["ids"], 32)
    sample = [int(offsets[ex]) for ex in range(32) if counts[ex] > 0]
    sample += [int(offsets[ex + 1]) - 1 for ex in range(32) if counts[ex] > 0]
    sample += list(rng.choice(32768, size=64, replace=False))
    _moe_block(rq, d, 16384, 2048, 4096, 32, 2, sample=np.unique(np.array(sample)))
