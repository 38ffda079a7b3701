"""GPU MoE grouped linear vs the oracle.

Stage by stage: the per-token (or per-permuted-row) quantization is bit-exact; every
permuted GEMM row is within the linear tolerance of the oracle evaluated on the GPU's own
quantized operand; the SiLU rows are within 1 FP16 ulp; the combined output is within 1
FP16 ulp of the oracle's combine of the GPU's permuted rows.  Ragged expert loads include
empty experts; the full-size Zipf workload (16384 tokens, top-2 of 32 experts) is checked
on every row, in the gated formulation the benchmark times.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, linear, moe, quant
from tests import parity
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu


def _quant_experts(rq, w16):
    w_q, w_s = rq.quant_weights(dev(w16))
    return w_q, w_s


def _check_rows_by_expert(y, a_q, a_s, src_of_row, rows, offsets, w_q, w_s):
    """linear.check of permuted output rows, one oracle call per expert."""
    experts = np.searchsorted(offsets, rows, side="right") - 1
    for ex in np.unique(experts):
        r = rows[experts == ex]
        src = src_of_row(r)
        ok, ratio, _ = linear.check(y[r], a_q[src], a_s[src], w_q[ex], w_s[ex])
        assert ok, (int(ex), ratio)


def _expert_ffn(d, t, k, f, e, top_k, sample=None):
    """Run the two grouped calls of an expert FFN and check every stage."""
    rq = require_gpu()
    ids = d["ids"].astype(np.int32)
    wgu_q, wgu_s = _quant_experts(rq, d["w_gu"])
    wdn_q, wdn_s = _quant_experts(rq, d["w_dn"])
    wgu_qh, wgu_sh = host(wgu_q), host(wgu_s)
    wdn_qh, wdn_sh = host(wdn_q), host(wdn_s)
    # weight quantization: every expert, a slice of rows each
    for ex in range(e):
        sl = slice(0, None) if sample is None else slice(0, 64)
        rq_, rs_ = quant.quantize_rows(d["w_gu"][ex][sl])
        assert np.array_equal(wgu_qh[ex][sl], rq_) and np.array_equal(wgu_sh[ex][sl], rs_)

    x, ids_d, tw = dev(d["x"]), dev(ids), dev(d["topk_w"])
    gu, dbg1 = rq.moe_grouped_linear(x, ids_d, wgu_q, wgu_s, "tokens", "none", "permuted", debug=True)
    gu_h, aq1, as1 = host(gu), host(dbg1["a_q"]), host(dbg1["a_scale"])
    xq, xs = quant.quantize_rows(d["x"])
    counts, offsets, perm, pos = moe.plan(ids, e)
    # the GEMM operand: permuted row r holds token perm[r] // top_k, quantized once per token
    tok = perm // top_k
    assert np.array_equal(aq1, xq[tok]) and np.array_equal(as1.view(np.uint32), xs[tok].view(np.uint32))

    rows = np.arange(t * top_k) if sample is None else np.asarray(sample)
    _check_rows_by_expert(gu_h, xq, xs, lambda r: perm[r] // top_k, rows, offsets, wgu_qh, wgu_sh)

    out, dbg2 = rq.moe_grouped_linear(gu, ids_d, wdn_q, wdn_s, "permuted", "silu_mul", "combined",
                                      topk_w=tw, debug=True)
    y_perm = rq.moe_grouped_linear(gu, ids_d, wdn_q, wdn_s, "permuted", "silu_mul", "permuted")
    out, h, aq2, as2, y_perm = host(out), host(dbg2["h"]), host(dbg2["a_q"]), host(dbg2["a_scale"]), host(y_perm)
    assert ulp_diff16(h[rows], ffn.silu_mul(gu_h[rows], f)).max() <= 1
    hq, hs = quant.quantize_rows(h[rows])
    assert np.array_equal(aq2[rows], hq) and np.array_equal(as2[rows].view(np.uint32), hs.view(np.uint32))
    _check_rows_by_expert(y_perm, aq2, as2, lambda r: r, rows, offsets, wdn_qh, wdn_sh)
    comb_ref = moe.combine(y_perm, pos, d["topk_w"])
    assert ulp_diff16(out, comb_ref).max() <= 1
    return counts


@pytest.mark.parametrize("t,k,f,e,top_k", [
    (37, 64, 48, 5, 2), (300, 128, 144, 8, 2), (129, 256, 272, 16, 1), (64, 48, 32, 6, 4),
    # the routing plan in three kernels: more than 8192 routed slots, or more than 256 experts
    (40000, 64, 32, 8, 2), (700, 64, 32, 300, 2),
])
def test_expert_ffn_small(t, k, f, e, top_k):
    case("moe t=%d k=%d f=%d e=%d top_k=%d" % (t, k, f, e, top_k))
    d = workloads.make(4, t=t, k=k, f=f, e=e, top_k=top_k)
    counts = _expert_ffn(d, t, k, f, e, top_k)
    assert (counts == 0).any()


def test_single_expert_equals_dense():
    rq = require_gpu()
    case("moe: all tokens on one expert")
    rng = np.random.default_rng(0)
    t, k, n, e = 200, 256, 160, 6
    x = workloads.acts_outliers(rng, t, k)
    w = workloads.weights(rng, (e, n, k))
    w_q, w_s = rq.quant_weights(dev(w))
    ids = np.full((t, 1), 4, np.int32)
    y = host(rq.moe_grouped_linear(dev(x), dev(ids), w_q, w_s))
    dense = host(rq.linear(dev(x), w_q[4].contiguous(), w_s[4].contiguous()))
    assert np.array_equal(y.view(np.uint16), dense.view(np.uint16))


def test_zero_tokens():
    rq = require_gpu()
    case("moe: T = 0")
    w_q = torch.zeros((4, 32, 64), dtype=torch.uint8, device="cuda")
    w_s = torch.ones((4, 32), dtype=torch.float32, device="cuda")
    y = rq.moe_grouped_linear(torch.zeros((0, 64), dtype=torch.float16, device="cuda"),
                              torch.zeros((0, 2), dtype=torch.int32, device="cuda"), w_q, w_s)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


def test_moe_determinism():
    rq = require_gpu()
    case("moe determinism")
    d = workloads.make(4, t=1000, k=256, f=128, e=8)
    w_q, w_s = rq.quant_weights(dev(d["w_gu"]))
    x, ids = dev(d["x"]), dev(d["ids"].astype(np.int32))
    a = host(rq.moe_grouped_linear(x, ids, w_q, w_s))
    b = host(rq.moe_grouped_linear(x, ids, w_q, w_s))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.slow
def test_moe_full_size_every_row():
    """16384 tokens, top-2 of 32 Zipf-loaded experts, F = 4096, as the benchmark runs it
    (gated gate/up, down with the combine, slab-layout expert weights), every permuted row
    checked expert by expert."""
    rq = require_gpu()
    d = workloads.make(4)
    counts, r_gu, r_dn = parity.moe_ffn_gated(rq, d["x"], d["ids"], d["topk_w"], d["w_gu"], d["w_dn"],
                                              "workload 4: MoE 16384 tokens, top-2 of 32, F = 4096", "slabs")
    assert (counts == 0).any()


@pytest.mark.parametrize("grid", [None, "5", "16"])
@pytest.mark.parametrize("tile", ["256x256", "64x256", "64x128", None])
def test_grouped_tile_shapes(monkeypatch, tile, grid):
    # 600 tokens, top-2 of 6 experts: about 200 rows per expert (256-row tiles by default);
    # a capped grid makes each workgroup walk many expert tiles
    case("moe tile=%s grid=%s" % (tile, grid))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    if grid is not None:
        monkeypatch.setenv("RQ_GEMM_GRID", grid)
    d = workloads.make(4, t=600, k=320, f=144, e=6)
    _expert_ffn(d, 600, 320, 144, 6, 2)


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
@pytest.mark.parametrize("t,k,f,e", [(300, 128, 64, 6), (600, 320, 160, 4)])
def test_gated_expert_ffn(monkeypatch, tile, t, k, f, e):
    """(TOKENS, GATE_SILU, PERMUTED) on interleaved expert weights writes exactly the h of the
    plain (TOKENS, NONE, PERMUTED) call followed by the down call's SiLU*up transform, and
    the down call on it (PERMUTED, NONE, COMBINED) matches the unfused FFN bit for bit."""
    rq = require_gpu()
    case("moe gated tile=%s t=%d k=%d f=%d e=%d" % (tile, t, k, f, e))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids, tw, x = dev(d["ids"].astype(np.int32)), dev(d["topk_w"]), dev(d["x"])
    wgu_q, wgu_s = rq.quant_weights(dev(d["w_gu"]))
    wdn_q, wdn_s = rq.quant_weights(dev(d["w_dn"]))
    order = torch.from_numpy(ffn.gate_up_order(f)).cuda()
    wgi_q, wgi_s = wgu_q[:, order].contiguous(), wgu_s[:, order].contiguous()
    h = rq.moe_grouped_linear(x, ids, wgi_q, wgi_s, "tokens", "gate_silu", "permuted")
    assert tuple(h.shape) == (2 * t, f)
    gu = rq.moe_grouped_linear(x, ids, wgu_q, wgu_s, "tokens", "none", "permuted")
    out_plain, dbg = rq.moe_grouped_linear(gu, ids, wdn_q, wdn_s, "permuted", "silu_mul", "combined",
                                           topk_w=tw, debug=True)
    assert np.array_equal(host(h).view(np.uint16), host(dbg["h"]).view(np.uint16))
    out = rq.moe_grouped_linear(h, ids, wdn_q, wdn_s, "permuted", "none", "combined", topk_w=tw)
    assert np.array_equal(host(out).view(np.uint16), host(out_plain).view(np.uint16))


@pytest.mark.parametrize("t,k,f,e", [(512, 2048, 4096, 32), (600, 320, 160, 6), (3000, 256, 128, 8)])
def test_plan_reuse_equals_fresh_plan(t, k, f, e):
    """The down call with RQ_MOE_PLAN_READY on the gate/up call's workspace gives the bytes of a
    down call that builds its own plan (the 512-token case: gate/up on 64-row tiles, down on
    256-row tiles, so the reused plan serves the other tile height)."""
    rq = require_gpu()
    case("moe plan reuse t=%d k=%d f=%d e=%d" % (t, k, f, e))
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids, tw, x = dev(d["ids"].astype(np.int32)), dev(d["topk_w"]), dev(d["x"])
    wgu = rq.quant_weights(dev(rq.interleave_gate_up(d["w_gu"])))
    wdn = rq.quant_weights(dev(d["w_dn"]))
    size = max(rq.moe_workspace_size(t, 2, e, 2 * f, k, "tokens", "gate_silu", "permuted"),
               rq.moe_workspace_size(t, 2, e, k, f, "permuted", "none", "combined"))
    shared = torch.empty(size, dtype=torch.uint8, device="cuda")
    h = rq.moe_grouped_linear(x, ids, *wgu, "tokens", "gate_silu", "permuted", workspace=shared)
    reused = host(rq.moe_grouped_linear(h, ids, *wdn, "permuted", "none", "combined", topk_w=tw,
                                        workspace=shared, plan_ready=True))
    fresh = host(rq.moe_grouped_linear(h, ids, *wdn, "permuted", "none", "combined", topk_w=tw))
    assert np.array_equal(reused.view(np.uint16), fresh.view(np.uint16))
    # and the permuted output too (the GEMM's tile table alone)
    yp_r = host(rq.moe_grouped_linear(h, ids, *wdn, "permuted", "none", "permuted", workspace=shared,
                                      plan_ready=True))
    yp_f = host(rq.moe_grouped_linear(h, ids, *wdn, "permuted", "none", "permuted"))
    assert np.array_equal(yp_r.view(np.uint16), yp_f.view(np.uint16))
