"""Sizes at the edges of the C ABI's limits, against the oracle: a long K that takes the
quantizer's two-pass path for rows wider than its register path (K = 65536) and a 1024-long
GEMM K loop; the largest expert count (E = 1024, most experts empty, the three-kernel routing
plan); one token routed to every expert of a small set (top_k = E)."""

import numpy as np
import pytest

import workloads
from oracle import moe, quant
from tests import parity
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k,wlayout", [(3, 64, 65536, "rows"), (5, 128, 65536, "slabs"), (70, 32, 24576, "rows")])
def test_long_k_linear(m, n, k, wlayout):
    rq = require_gpu()
    case("long-K linear m=%d n=%d k=%d %s" % (m, n, k, wlayout))
    d = workloads.make(1, m=m, k=k, n=n)
    wq, ws = rq.quant_weights(dev(d["w"]))
    wt = rq.pack_weights(wq) if wlayout == "slabs" else wq
    y, dbg = rq.linear(dev(d["x"]), wt, ws, debug=True, wlayout=wlayout)
    wq_h, ws_h = host(wq), host(ws)
    parity.check_quant(wq_h, ws_h, d["w"])
    xq, xs = parity.check_quant(host(dbg["a_q"]), host(dbg["a_scale"]), d["x"])
    parity.check_rows(host(y), xq, xs, wq_h, ws_h)


def _moe_check(rq, t, e, top_k, n, k, ids):
    rng = np.random.default_rng(t + e)
    x = workloads.acts_outliers(rng, t, k)
    w = workloads.weights(rng, (e, n, k))
    logits = rng.standard_normal((t, top_k))
    tw = (np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)).astype(np.float16)
    wq, ws = rq.quant_weights(dev(w))
    ids_d, x_d = dev(ids), dev(x)
    y, dbg = rq.moe_grouped_linear(x_d, ids_d, wq, ws, "tokens", "none", "combined", topk_w=dev(tw), debug=True)
    y_perm = host(rq.moe_grouped_linear(x_d, ids_d, wq, ws, "tokens", "none", "permuted"))
    counts, offsets, perm, pos = moe.plan(ids, e)
    xq, xs = quant.quantize_rows(x)
    assert np.array_equal(host(dbg["a_q"]), xq[perm // top_k])
    ok, ratio = moe.grouped_linear_check(y_perm, xq, xs, moe.IN_TOKENS, ids, host(wq), host(ws))
    assert ok, ratio
    assert ulp_diff16(host(y), moe.combine(y_perm, pos, tw)).max() <= 1
    return counts


def test_most_experts_empty_at_the_expert_limit():
    rq = require_gpu()
    t, e, top_k, n, k = 300, 1024, 2, 64, 128
    case("moe E=%d t=%d" % (e, t))
    rng = np.random.default_rng(11)
    ids = np.argsort(rng.random((t, e)), axis=1)[:, :top_k].astype(np.int32)
    counts = _moe_check(rq, t, e, top_k, n, k, ids)
    assert (counts == 0).sum() > e // 2


def test_top_k_equals_expert_count():
    rq = require_gpu()
    t, e, n, k = 97, 4, 96, 256
    case("moe top_k = E = %d, t=%d" % (e, t))
    rng = np.random.default_rng(12)
    ids = np.argsort(rng.random((t, e)), axis=1).astype(np.int32)  # every token to every expert
    counts = _moe_check(rq, t, e, e, n, k, ids)
    assert (counts == t).all()
