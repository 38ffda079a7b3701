"""Slab weight layout on the GPU.

The packing kernel must write exactly the permutation of ``oracle.layout`` (bit for bit), and
every linear on packed weights must give, bit for bit, the result of the same call on the row
layout - the GEMM only finds the same bytes at other addresses, so its LDS contents and its
accumulation order are unchanged.  The row layout's parity against the oracle is checked by
the other GPU tests; here the cases span every tile shape, N that ends inside a tile (the
tile's rows past N then read the next slab's first rows, which feed only columns that are
never stored), split-K, the gated output, the SiLU*up input, weight scales per tensor and per
128 x 128 block, E5M2 activations and the grouped MoE path; one case is also checked against
the oracle directly.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import layout
from tests import parity
from tests.gpu_util import case, dev, host, require_gpu

pytestmark = pytest.mark.gpu

TILES = [None, "256x256", "256x192", "256x128", "128x128", "64x128", "64x256"]


def _bits(t):
    return host(t).view(np.uint16)


@pytest.mark.parametrize("shape", [(16, 64), (2, 272, 192), (3, 384, 2048), (32, 2048, 4096)])
def test_pack_matches_oracle(shape):
    rq = require_gpu()
    case("pack %r" % (shape,))
    rng = np.random.default_rng(sum(shape))
    w = rng.integers(0, 256, size=shape, dtype=np.uint8)
    got = host(rq.pack_weights(dev(w))).reshape(-1)
    assert np.array_equal(got, layout.pack_slabs(w))


def test_pack_rejects_unaligned_and_in_place():
    rq = require_gpu()
    w = torch.zeros((128, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(rq.RqError):
        rq.pack_weights(torch.zeros((128, 48), dtype=torch.uint8, device="cuda"))
    with pytest.raises(rq.RqError):
        rq.pack_weights(w, out=w)


def _linear_pair(rq, x, w16, **kw):
    wq, ws = rq.quant_weights(dev(w16), wscale=kw.get("wscale", "channel"))
    wp = rq.pack_weights(wq)
    y_rows = rq.linear(x, wq, ws, **kw)
    y_slabs = rq.linear(x, wp, ws, wlayout="slabs", **kw)
    return y_rows, y_slabs


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(300, 400, 320), (64, 512, 512), (1000, 1168, 1024), (17, 48, 128)])
def test_linear_slabs_equal_rows(monkeypatch, tile, m, n, k):
    rq = require_gpu()
    case("linear slabs tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    d = workloads.make(1, m=m, k=k, n=n)
    y_rows, y_slabs = _linear_pair(rq, dev(d["x"]), d["w"])
    assert np.array_equal(_bits(y_rows), _bits(y_slabs))


@pytest.mark.parametrize("m,n,k", [(512, 2048, 8192), (300, 6144, 4096), (1, 512, 8192), (64, 272, 4096)])
def test_split_k_slabs_equal_rows(m, n, k):
    """Few rows and long K: the call cuts K into parts, each starting k0 * N bytes into the
    matrix."""
    rq = require_gpu()
    case("split-K slabs m=%d n=%d k=%d" % (m, n, k))
    assert rq.linear_workspace_size(m, k, n=n) > rq.linear_workspace_size(m, k)  # the call splits
    d = workloads.make(1, m=m, k=k, n=n)
    y_rows, y_slabs = _linear_pair(rq, dev(d["x"]), d["w"])
    assert np.array_equal(_bits(y_rows), _bits(y_slabs))


@pytest.mark.parametrize("act", ["gate_silu", "silu_mul"])
@pytest.mark.parametrize("m,n,k", [(512, 1024, 2048), (96, 1088, 8192), (4096, 512, 256)])
def test_ffn_activations_slabs_equal_rows(act, m, n, k):
    rq = require_gpu()
    case("linear slabs act=%s m=%d n=%d k=%d" % (act, m, n, k))
    rng = np.random.default_rng(m + n + k)
    x = workloads.acts_outliers(rng, m, 2 * k if act == "silu_mul" else k)
    w = workloads.weights(rng, (n, k))
    y_rows, y_slabs = _linear_pair(rq, dev(x), w, act=act)
    assert np.array_equal(_bits(y_rows), _bits(y_slabs))


@pytest.mark.parametrize("wscale,afmt", [("tensor", "e4m3"), ("block128", "e4m3"), ("channel", "e5m2"),
                                         ("block128", "e5m2")])
@pytest.mark.parametrize("m", [200, 4096])
def test_scale_formats_slabs_equal_rows(wscale, afmt, m):
    rq = require_gpu()
    case("linear slabs wscale=%s afmt=%s m=%d" % (wscale, afmt, m))
    d = workloads.make(1, m=m, k=1024, n=640)
    y_rows, y_slabs = _linear_pair(rq, dev(d["x"]), d["w"], wscale=wscale, afmt=afmt)
    assert np.array_equal(_bits(y_rows), _bits(y_slabs))


def test_slab_linear_against_oracle():
    """One packed-weight linear checked against the oracle row by row (the tolerance of the
    row-layout tests), with a ragged M tail and N ending inside a 256-column tile."""
    rq = require_gpu()
    m, n, k = 1100, 656, 1536
    case("linear slabs vs oracle m=%d n=%d k=%d" % (m, n, k))
    d = workloads.make(1, m=m, k=k, n=n)
    wq, ws = rq.quant_weights(dev(d["w"]))
    y, dbg = rq.linear(dev(d["x"]), rq.pack_weights(wq), ws, wlayout="slabs", debug=True)
    wq_h, ws_h = host(wq), host(ws)
    parity.check_quant(wq_h, ws_h, d["w"])
    xq, xs = parity.check_quant(host(dbg["a_q"]), host(dbg["a_scale"]), d["x"])
    parity.check_rows(host(y), xq, xs, wq_h, ws_h)


@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
@pytest.mark.parametrize("t,k,f,e", [(600, 320, 128, 6), (2000, 512, 384, 16)])
def test_moe_slabs_equal_rows(monkeypatch, tile, t, k, f, e):
    """The expert FFN as the benchmark chains it - gated gate/up to permuted rows, then the
    down call with the combine reusing the plan - on packed and on row-layout expert weights."""
    rq = require_gpu()
    case("moe slabs tile=%s t=%d k=%d f=%d e=%d" % (tile, t, k, f, e))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids, tw, x = dev(d["ids"].astype(np.int32)), dev(d["topk_w"]), dev(d["x"])
    wgu_q, wgu_s = rq.quant_weights(dev(d["w_gu"]))
    wdn_q, wdn_s = rq.quant_weights(dev(d["w_dn"]))
    wgu_p, wdn_p = rq.pack_weights(wgu_q), rq.pack_weights(wdn_q)
    outs = {}
    for wl, (gq, dq) in {"rows": (wgu_q, wdn_q), "slabs": (wgu_p, wdn_p)}.items():
        ws = torch.empty(rq.moe_workspace_size(t, 2, e, 2 * f, k, "tokens", "gate_silu", "permuted") +
                         rq.moe_workspace_size(t, 2, e, k, f, "permuted", "none", "combined"),
                         dtype=torch.uint8, device="cuda")
        h = rq.moe_grouped_linear(x, ids, gq, wgu_s, "tokens", "gate_silu", "permuted", workspace=ws, wlayout=wl)
        y = rq.moe_grouped_linear(h, ids, dq, wdn_s, "permuted", "none", "combined", topk_w=tw, workspace=ws,
                                  plan_ready=True, wlayout=wl)
        outs[wl] = (_bits(h), _bits(y))
    assert np.array_equal(outs["rows"][0], outs["slabs"][0])
    assert np.array_equal(outs["rows"][1], outs["slabs"][1])


@pytest.mark.parametrize("wscale,afmt", [("block128", "e4m3"), ("tensor", "e4m3"), ("channel", "e5m2")])
@pytest.mark.parametrize("tile", [None, "256x256", "64x256"])
def test_moe_scale_formats_slabs_equal_rows(monkeypatch, tile, wscale, afmt):
    """The grouped GEMM's scale and activation-format variants (the benchmark times the
    block-scaled expert FFN on slab-layout weights) give the row layout's bytes."""
    rq = require_gpu()
    case("moe slabs wscale=%s afmt=%s tile=%s" % (wscale, afmt, tile))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    t, k, f, e = 700, 256, 256, 6
    d = workloads.make(4, t=t, k=k, f=f, e=e)
    ids, tw, x = dev(d["ids"].astype(np.int32)), dev(d["topk_w"]), dev(d["x"])
    wgu_q, wgu_s = rq.quant_weights(dev(rq.interleave_gate_up(d["w_gu"])), wscale=wscale)
    wdn_q, wdn_s = rq.quant_weights(dev(d["w_dn"]), wscale=wscale)
    outs = {}
    for wl, (gq, dq) in {"rows": (wgu_q, wdn_q), "slabs": (rq.pack_weights(wgu_q), rq.pack_weights(wdn_q))}.items():
        h = rq.moe_grouped_linear(x, ids, gq, wgu_s, "tokens", "gate_silu", "permuted", wscale=wscale, afmt=afmt,
                                  wlayout=wl)
        y = rq.moe_grouped_linear(h, ids, dq, wdn_s, "permuted", "none", "combined", topk_w=tw, wscale=wscale,
                                  afmt=afmt, wlayout=wl)
        outs[wl] = (_bits(h), _bits(y))
    assert np.array_equal(outs["rows"][0], outs["slabs"][0])
    assert np.array_equal(outs["rows"][1], outs["slabs"][1])
