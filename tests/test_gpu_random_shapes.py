"""Seeded random shapes and options through the linear and the MoE grouped linear, against the
oracle.

Each case draws its sizes (rows from 1, widths from 16, ragged against every tile), the weight
scale granularity, the activation format, the weight layout and, for the MoE, the expert count,
top-k, routing (distinct random experts per token, so some experts may be empty), input and
output layouts.  Checks as everywhere: weight and activation bytes and scales bit-exact,
every output row within the linear tolerance of the oracle evaluated on the GPU's own quantized
operand, the combined output within 1 FP16 ulp of the oracle's combine of the GPU's permuted
rows.
"""

import numpy as np
import pytest

import workloads
from oracle import moe, quant, wscale
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu

GRAN = {"channel": wscale.CHANNEL, "tensor": wscale.TENSOR, "block128": wscale.BLOCK128}


def _bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("seed", range(24))
def test_random_linear(seed):
    rq = require_gpu()
    rng = np.random.default_rng(9100 + seed)
    gran = ("channel", "tensor", "block128")[seed % 3]
    afmt = ("e4m3", "e5m2")[(seed // 3) % 2]
    if gran == "block128":
        n, k = 128 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 13))
    else:
        n, k = 16 * int(rng.integers(1, 81)), 16 * int(rng.integers(1, 129))
    m = int(rng.integers(1, 800))
    wlayout = "slabs" if k % 64 == 0 and seed % 2 == 0 else "rows"
    case("random linear seed=%d m=%d n=%d k=%d %s %s %s" % (seed, m, n, k, gran, afmt, wlayout))
    x = workloads.acts_outliers(rng, m, k)
    w = workloads.weights(rng, (n, k))
    wq, ws = rq.quant_weights(dev(w), wscale=gran)
    q_ref, s_ref = wscale.quantize(w, GRAN[gran])
    assert np.array_equal(host(wq), q_ref)
    assert np.array_equal(_bits32(host(ws)).ravel(), _bits32(s_ref).ravel())
    wt = rq.pack_weights(wq) if wlayout == "slabs" else wq
    y, dbg = rq.linear(dev(x), wt, ws, debug=True, wscale=gran, afmt=afmt, wlayout=wlayout)
    xq, xs = quant.quantize_rows(x, fmt=afmt)
    assert np.array_equal(host(dbg["a_q"]), xq)
    assert np.array_equal(_bits32(host(dbg["a_scale"])), _bits32(xs))
    ok, ratio, _ = wscale.check(host(y), xq, xs, q_ref, s_ref, GRAN[gran], a_fmt=afmt)
    assert ok, ratio


@pytest.mark.parametrize("seed", range(24))
def test_random_moe(seed):
    rq = require_gpu()
    rng = np.random.default_rng(9300 + seed)
    e = int(rng.integers(1, 41))
    top_k = int(rng.integers(1, min(4, e) + 1))
    t = int(rng.integers(1, 700))
    n, k = 16 * int(rng.integers(1, 41)), 16 * int(rng.integers(1, 97))
    in_layout = ("tokens", "permuted")[seed % 2]
    out_layout = ("permuted", "combined")[(seed // 2) % 2]
    wlayout = "slabs" if k % 64 == 0 and seed % 3 == 0 else "rows"
    case("random moe seed=%d t=%d e=%d top_k=%d n=%d k=%d %s %s %s" % (seed, t, e, top_k, n, k, in_layout,
                                                                       out_layout, wlayout))
    ids = np.argsort(rng.random((t, e)), axis=1)[:, :top_k].astype(np.int32)  # distinct experts per token
    logits = rng.standard_normal((t, top_k))
    tw = (np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)).astype(np.float16)
    r = t * top_k
    x = workloads.acts_outliers(rng, t if in_layout == "tokens" else r, k)
    w = workloads.weights(rng, (e, n, k))
    wq, ws = rq.quant_weights(dev(w))
    wq_h, ws_h = host(wq), host(ws)
    q_ref, s_ref = quant.quantize_rows(w.reshape(e * n, k))
    assert np.array_equal(wq_h.reshape(e * n, k), q_ref)
    wt = rq.pack_weights(wq) if wlayout == "slabs" else wq
    ids_d, tw_d, x_d = dev(ids), dev(tw), dev(x)
    y, dbg = rq.moe_grouped_linear(x_d, ids_d, wt, ws, in_layout, "none", out_layout,
                                   topk_w=tw_d if out_layout == "combined" else None, debug=True, wlayout=wlayout)
    y_perm = y if out_layout == "permuted" else rq.moe_grouped_linear(x_d, ids_d, wt, ws, in_layout, "none",
                                                                    "permuted", wlayout=wlayout)
    counts, offsets, perm, pos = moe.plan(ids, e)
    xq, xs = quant.quantize_rows(x)
    src = perm // top_k if in_layout == "tokens" else np.arange(r)
    assert np.array_equal(host(dbg["a_q"]), xq[src])
    assert np.array_equal(_bits32(host(dbg["a_scale"])), _bits32(xs[src]))
    il = moe.IN_TOKENS if in_layout == "tokens" else moe.IN_PERMUTED
    ok, ratio = moe.grouped_linear_check(host(y_perm), xq, xs, il, ids, wq_h, ws_h)
    assert ok, ratio
    if out_layout == "combined":
        assert ulp_diff16(host(y), moe.combine(host(y_perm), pos, tw)).max() <= 1
