"""Stage-by-stage parity checks of whole FFN chains against the oracle (GPU tests only).

Every output row is compared, in row chunks so that the oracle's float64 products stay a
few GB at the full workload sizes.  The chains run exactly as the benchmark runs them:

* dense FFN: the gate/up linear on interleaved weights writes h = silu(g) * u from its
  epilogue (``act='gate_silu'``), the down linear quantizes h per token;
* expert FFN: the grouped gate/up call (TOKENS, GATE_SILU, PERMUTED) and the grouped down
  call (PERMUTED, NONE, COMBINED) on the same workspace, reusing the gate/up call's routing
  plan.

Each gated call is also compared bit for bit with the unfused formulation (plain gate/up
output, then the SiLU*up input transform of the down call), whose intermediate the oracle
checks directly: g and u within the linear tolerance, h within 1 FP16 ulp of the oracle's
SiLU of the GPU's own g and u, the quantized h bit-exact.
"""

import concurrent.futures
import os

import numpy as np
import torch

from oracle import ffn, linear, moe, quant
from tests.gpu_util import case, dev, host, ulp_diff16

CHUNK = 1024


def check_rows(y, xq, xs, wq, ws, rows=None, chunk=CHUNK):
    """``oracle.linear.check`` over every row (or ``rows``), in chunks; returns the worst
    ratio |d| / tol and asserts it is at most 1."""
    idx = np.arange(y.shape[0]) if rows is None else np.asarray(rows)
    worst = 0.0
    for lo in range(0, idx.size, chunk):
        r = idx[lo:lo + chunk]
        ok, ratio, _ = linear.check(y[r], xq[r], xs[r], wq, ws)
        worst = max(worst, ratio)
        assert ok, "rows %d..%d: max |d|/tol = %.3f" % (int(r[0]), int(r[-1]), ratio)
    return worst


def _quantize_blocks(rows16, block=1024):
    """The oracle's row quantizer over row blocks on a thread pool (numpy releases the
    interpreter lock inside its array operations); rows are independent, so the result is
    the one-call result."""
    rows16 = np.asarray(rows16)
    flat = rows16.reshape(-1, rows16.shape[-1])
    starts = list(range(0, flat.shape[0], block))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda lo: quant.quantize_rows(flat[lo:lo + block]), starts))
    q = np.concatenate([p[0] for p in parts]) if parts else np.zeros(flat.shape, np.uint8)
    s = np.concatenate([p[1] for p in parts]) if parts else np.zeros(flat.shape[0], np.float32)
    return q.reshape(rows16.shape), s.reshape(rows16.shape[:-1])


def check_quant(aq, a_s, rows16):
    """Quantized bytes and scales bit-exact against the oracle's row quantizer (any leading
    dimensions: a weight stack [E][N][K] is E * N independent rows)."""
    q, s = _quantize_blocks(rows16)
    assert np.array_equal(a_s.view(np.uint32), s.view(np.uint32)), "scales differ"
    assert np.array_equal(aq, q), "quantized bytes differ"
    return q, s


def _packed(rq, wq, wlayout):
    """The weights as the call takes them: packed offline for the slab layout."""
    return rq.pack_weights(wq) if wlayout == "slabs" else wq


def linear_all_rows(rq, x16, w16, label, wlayout="rows"):
    """One plain linear: weight and activation bytes bit-exact, every output row within
    the tolerance.  Returns the GPU output (host) and the worst ratio."""
    case(label)
    wq, ws = rq.quant_weights(dev(w16))
    y, dbg = rq.linear(dev(x16), _packed(rq, wq, wlayout), ws, debug=True, wlayout=wlayout)
    wq_h, ws_h = host(wq), host(ws)
    check_quant(wq_h, ws_h, w16)
    xq, xs = check_quant(host(dbg["a_q"]), host(dbg["a_scale"]), x16)
    y = host(y)
    return y, check_rows(y, xq, xs, wq_h, ws_h)


def dense_ffn_gated(rq, x16, w_gu16, w_dn16, label, wlayout="rows"):
    """The dense FFN chain as the benchmark runs it (gated gate/up and down on weights in
    ``wlayout``), checked stage by stage."""
    f = w_gu16.shape[0] // 2
    case(label + ": gate/up, unfused and gated")
    wgu_q, wgu_s = rq.quant_weights(dev(w_gu16))
    order = torch.from_numpy(ffn.gate_up_order(f)).cuda()
    x = dev(x16)
    # unfused gate/up [g | u], checked on every row
    gu, dbg = rq.linear(x, wgu_q, wgu_s, debug=True)
    wgu_qh, wgu_sh = host(wgu_q), host(wgu_s)
    check_quant(wgu_qh, wgu_sh, w_gu16)
    xq, xs = check_quant(host(dbg["a_q"]), host(dbg["a_scale"]), x16)
    gu_h = host(gu)
    r_gu = check_rows(gu_h, xq, xs, wgu_qh, wgu_sh)
    # gated gate/up on interleaved weights (quantized from interleaved FP16 rows, as offline)
    wgi_q, wgi_s = rq.quant_weights(dev(rq.interleave_gate_up(w_gu16)))
    assert torch.equal(wgi_q, wgu_q[order]) and torch.equal(wgi_s, wgu_s[order])
    h = rq.linear(x, _packed(rq, wgi_q, wlayout), wgi_s, act="gate_silu", wlayout=wlayout)
    case(label + ": down")
    wdn_q, wdn_s = rq.quant_weights(dev(w_dn16))
    _, dbg_u = rq.linear(gu, wdn_q, wdn_s, act="silu_mul", debug=True)
    h_h = host(h)
    assert np.array_equal(h_h.view(np.uint16), host(dbg_u["h"]).view(np.uint16)), "gated h != unfused h"
    assert ulp_diff16(h_h, ffn.silu_mul(gu_h, f)).max() <= 1
    # down on the gated h, every row
    y, dbg_d = rq.linear(h, _packed(rq, wdn_q, wlayout), wdn_s, debug=True, wlayout=wlayout)
    wdn_qh, wdn_sh = host(wdn_q), host(wdn_s)
    check_quant(wdn_qh, wdn_sh, w_dn16)
    hq, hs = check_quant(host(dbg_d["a_q"]), host(dbg_d["a_scale"]), h_h)
    r_dn = check_rows(host(y), hq, hs, wdn_qh, wdn_sh)
    return r_gu, r_dn


def _check_experts(y_perm, aq, a_s, src_of_row, offsets, wq, ws, chunk=CHUNK):
    """linear.check of every permuted row, expert by expert (chunked)."""
    worst = 0.0
    for ex in range(wq.shape[0]):
        lo, hi = int(offsets[ex]), int(offsets[ex + 1])
        for c in range(lo, hi, chunk):
            r = np.arange(c, min(hi, c + chunk))
            src = src_of_row(r)
            ok, ratio, _ = linear.check(y_perm[r], aq[src], a_s[src], wq[ex], ws[ex])
            worst = max(worst, ratio)
            assert ok, "expert %d rows %d..%d: max |d|/tol = %.3f" % (ex, int(r[0]), int(r[-1]), ratio)
    return worst


def moe_ffn_gated(rq, x16, ids, topk_w, w_gu16, w_dn16, label, wlayout="rows"):
    """The expert FFN as the benchmark runs it (gated gate/up, then down with the combine
    reusing the plan, on expert weights in ``wlayout``), checked stage by stage on every row."""
    e, f2, k = w_gu16.shape
    f = f2 // 2
    t, top_k = ids.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    counts, offsets, perm, pos = moe.plan(ids, e)
    ids_d, tw, x = dev(ids), dev(topk_w), dev(x16)
    case(label + ": expert gate/up, unfused")
    wgu_q, wgu_s = rq.quant_weights(dev(w_gu16))
    wgu_qh, wgu_sh = host(wgu_q), host(wgu_s)
    check_quant(wgu_qh, wgu_sh, w_gu16)
    gu, dbg1 = rq.moe_grouped_linear(x, ids_d, wgu_q, wgu_s, "tokens", "none", "permuted", debug=True)
    gu_h, aq1, as1 = host(gu), host(dbg1["a_q"]), host(dbg1["a_scale"])
    xq, xs = _quantize_blocks(x16)
    tok = perm // top_k
    assert np.array_equal(aq1, xq[tok]) and np.array_equal(as1.view(np.uint32), xs[tok].view(np.uint32))
    r_gu = _check_experts(gu_h, xq, xs, lambda r: perm[r] // top_k, offsets, wgu_qh, wgu_sh)
    case(label + ": expert gate/up, gated")
    order = torch.from_numpy(ffn.gate_up_order(f)).cuda()
    wgi_q, wgi_s = rq.quant_weights(dev(rq.interleave_gate_up(w_gu16)))
    assert torch.equal(wgi_q, wgu_q[:, order]) and torch.equal(wgi_s, wgu_s[:, order])
    # as timed: one workspace for both calls, the down call reusing the gate/up call's plan
    shared = torch.empty(max(rq.moe_workspace_size(t, top_k, e, f2, k, "tokens", "gate_silu", "permuted"),
                             rq.moe_workspace_size(t, top_k, e, k, f, "permuted", "none", "combined")),
                         dtype=torch.uint8, device="cuda")
    h = rq.moe_grouped_linear(x, ids_d, _packed(rq, wgi_q, wlayout), wgi_s, "tokens", "gate_silu", "permuted",
                              workspace=shared, wlayout=wlayout)
    case(label + ": expert down, unfused and gated")
    wdn_q, wdn_s = rq.quant_weights(dev(w_dn16))
    out_u, dbg_u = rq.moe_grouped_linear(gu, ids_d, wdn_q, wdn_s, "permuted", "silu_mul", "combined",
                                         topk_w=tw, debug=True)
    h_h = host(h)
    assert np.array_equal(h_h.view(np.uint16), host(dbg_u["h"]).view(np.uint16)), "gated h != unfused h"
    assert ulp_diff16(h_h, ffn.silu_mul(gu_h, f)).max() <= 1
    wdn_t = _packed(rq, wdn_q, wlayout)
    out, dbg2 = rq.moe_grouped_linear(h, ids_d, wdn_t, wdn_s, "permuted", "none", "combined",
                                      topk_w=tw, debug=True, workspace=shared, plan_ready=True, wlayout=wlayout)
    out_h = host(out)
    assert np.array_equal(out_h.view(np.uint16), host(out_u).view(np.uint16)), "gated FFN != unfused FFN"
    wdn_qh, wdn_sh = host(wdn_q), host(wdn_s)
    check_quant(wdn_qh, wdn_sh, w_dn16)
    hq, hs = check_quant(host(dbg2["a_q"]), host(dbg2["a_scale"]), h_h)
    y_perm = host(rq.moe_grouped_linear(h, ids_d, wdn_t, wdn_s, "permuted", "none", "permuted", wlayout=wlayout))
    r_dn = _check_experts(y_perm, hq, hs, lambda r: r, offsets, wdn_qh, wdn_sh)
    assert ulp_diff16(out_h, moe.combine(y_perm, pos, topk_w)).max() <= 1
    return counts, r_gu, r_dn
