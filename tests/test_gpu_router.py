"""GPU MoE router (FP16 gate logits, top-k selection, softmax weights) vs the oracle.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1: the FP16 routing gate whose top-k
result feeds the MoE grouped GEMM.  The FP32 logits must lie within the FP32-accumulation
bound of the oracle's; the selection is an integer decision taken on the GPU's own FP32
logits, so it must equal the oracle's selection on those same values exactly, and agree with
the oracle's float64 selection wherever the k-th and (k+1)-th logits are farther apart than
the bound; the weights must be within 1 FP16 ulp of the oracle's softmax of the GPU logits.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import moe, quant, router
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu


def _inputs(rng, t, k, e):
    x = workloads.acts_channel_lognormal(rng, t, k)
    w = (rng.standard_normal((e, k)) / np.sqrt(k)).astype(np.float16)
    return x, w


def _check(x, w, top_k, ids, wts, lg):
    ref_lg = router.logits(x, w)
    bound = router.logit_error_bound(x, w)
    assert np.all(np.abs(lg.astype(np.float64) - ref_lg) <= bound)
    own = router.select(lg.astype(np.float64), top_k)
    assert np.array_equal(ids, own)
    assert ulp_diff16(wts, router.weights(lg.astype(np.float64), own)).max() <= 1
    # against the float64 selection where it is unambiguous
    srt = np.sort(ref_lg, axis=1)[:, ::-1]
    if top_k < ref_lg.shape[1]:
        clear = (srt[:, top_k - 1] - srt[:, top_k]) > 2 * bound.max(axis=1)
        ref_ids = router.select(ref_lg, top_k)
        assert np.array_equal(np.sort(ids[clear], axis=1), np.sort(ref_ids[clear], axis=1))
        return int(clear.sum())
    return ids.shape[0]


@pytest.mark.parametrize("t,k,e,top_k", [
    (1, 64, 32, 2), (100, 2048, 32, 2), (64, 128, 32, 1), (300, 512, 20, 3), (77, 256, 7, 4), (33, 2048, 32, 4),
])
def test_router_small(t, k, e, top_k):
    rq = require_gpu()
    case("router t=%d k=%d e=%d top_k=%d" % (t, k, e, top_k))
    rng = np.random.default_rng(t + k + e)
    x, w = _inputs(rng, t, k, e)
    ids, wts, lg = rq.router_topk(dev(x), dev(w), top_k, logits=True)
    _check(x, w, top_k, host(ids), host(wts), host(lg))


def test_ties_go_to_the_lower_expert():
    rq = require_gpu()
    case("router ties")
    rng = np.random.default_rng(7)
    x, w = _inputs(rng, 64, 256, 32)
    w[9] = w[3]                                               # experts 3 and 9 tie exactly
    w[20] = w[3]
    x[:, :] = np.abs(x)
    w[3] = np.abs(w[3]) + np.float16(0.01)                    # and win by a clear margin
    w[9], w[20] = w[3], w[3]
    ids, wts, lg = rq.router_topk(dev(x), dev(w), 3, logits=True)
    ids = host(ids)
    assert np.all(ids == np.array([3, 9, 20])), ids[:4]
    assert np.all(host(wts) == np.float16(1.0 / 3.0))


def test_router_feeds_the_grouped_linear():
    """The router's ids and weights drive a combined MoE call whose result matches the oracle's
    chain from the same routing."""
    rq = require_gpu()
    case("router -> moe")
    rng = np.random.default_rng(8)
    t, k, n, e = 200, 256, 128, 8
    x, w = _inputs(rng, t, k, e)
    ids, wts = rq.router_topk(dev(x), dev(w), 2)
    wq, ws = rq.quant_weights(dev(workloads.weights(rng, (e, n, k))))
    out, dbg = rq.moe_grouped_linear(dev(x), ids, wq, ws, "tokens", "none", "combined", topk_w=wts, debug=True)
    ids_h, wts_h = host(ids), host(wts)
    ref = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids_h, host(wq), host(ws), moe.OUT_COMBINED, wts_h)
    xq, _ = quant.quantize_rows(x)
    assert np.array_equal(host(dbg["a_q"]), xq[ref["perm"] // 2])
    y_perm = host(rq.moe_grouped_linear(dev(x), ids, wq, ws, "tokens", "none", "permuted"))
    ok, ratio = moe.grouped_linear_check(y_perm, xq, quant.quantize_rows(x)[1], moe.IN_TOKENS, ids_h, host(wq),
                                         host(ws))
    assert ok, ratio
    assert ulp_diff16(host(out), moe.combine(y_perm, ref["pos"], wts_h)).max() <= 1


def test_argument_errors():
    rq = require_gpu()
    case("router argument errors")
    x = dev(np.zeros((4, 128), np.float16))
    with pytest.raises(rq.RqError):
        rq.router_topk(x, dev(np.zeros((33, 128), np.float16)), 2)       # E > 32
    with pytest.raises(rq.RqError):
        rq.router_topk(x, dev(np.zeros((8, 128), np.float16)), 5)        # top_k > 4
    with pytest.raises(rq.RqError):
        rq.router_topk(dev(np.zeros((4, 96), np.float16)), dev(np.zeros((8, 96), np.float16)), 2)  # K % 64


@pytest.mark.slow
def test_router_full_size():
    """The MoE workload's shape: 16384 tokens x 2048, 32 experts, top-2."""
    rq = require_gpu()
    case("router full size 16384 x 2048, E = 32")
    rng = np.random.default_rng(9)
    x, w = _inputs(rng, 16384, 2048, 32)
    ids, wts, lg = rq.router_topk(dev(x), dev(w), 2, logits=True)
    clear = _check(x, w, 2, host(ids), host(wts), host(lg))
    assert clear > 16000
