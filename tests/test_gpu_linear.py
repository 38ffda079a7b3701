"""GPU W8A8 linear vs the oracle.

Quantized activations (the bytes and scales the GEMM actually consumed, returned through
the debug outputs) must equal the oracle's bit for bit; FP16 outputs must lie within

    |y - y_ref| <= 2 ulp16(y_ref) + 1e-3 * s_x[m] * s_w[n] * sum_k |dec(x_q) dec(w_q)|

of the oracle's exactly accumulated result (``oracle.linear.check``).  Small shapes span
several 128-wide tiles with ragged M, N and K tails; the full-size workloads (dense 64 x
512 x 512, attention QKV/O at 4096 tokens, the FFN at 4096 tokens) are checked on every
quantized byte and on sampled output rows, in the same launch configuration the
benchmark uses.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, linear, quant
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff16

pytestmark = pytest.mark.gpu


def _run_linear(x16, w16, act="none", rows=None):
    rq = require_gpu()
    w_q, w_s = rq.quant_weights(dev(w16))
    y, dbg = rq.linear(dev(x16), w_q, w_s, act=act, debug=True)
    return host(y), {k: (host(v) if v is not None else None) for k, v in dbg.items()}, host(w_q), host(w_s)


def _check(x16, w16, act="none", sample_rows=None):
    y, dbg, wq, ws = _run_linear(x16, w16, act)
    wq_ref, ws_ref = quant.quantize_rows(w16)
    assert np.array_equal(wq, wq_ref) and np.array_equal(ws.view(np.uint32), ws_ref.view(np.uint32))
    if act == "silu_mul":
        k = w16.shape[1]
        assert ulp_diff16(dbg["h"], ffn.silu_mul(x16, k)).max() <= 1
        rows_in = dbg["h"]
    else:
        rows_in = x16
    xq_ref, sx_ref = quant.quantize_rows(rows_in)
    assert np.array_equal(dbg["a_scale"].view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(dbg["a_q"], xq_ref)
    r = np.arange(x16.shape[0]) if sample_rows is None else sample_rows
    ok, ratio, _ = linear.check(y[r], xq_ref[r], sx_ref[r], wq_ref, ws_ref)
    assert ok, "max |d|/tol = %.3f" % ratio
    return ratio


@pytest.mark.parametrize("m,n,k", [
    (1, 16, 16), (3, 48, 112), (16, 128, 128), (64, 512, 512), (130, 144, 144),
    (257, 272, 528), (200, 384, 2048), (129, 256, 8192), (5, 1040, 272),
])
def test_small_shapes(m, n, k):
    case("linear m=%d n=%d k=%d" % (m, n, k))
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    x = workloads.acts_outliers(rng, m, k)
    w = workloads.weights(rng, (n, k))
    _check(x, w)


@pytest.mark.parametrize("m,n,k", [(5, 32, 64), (130, 144, 528), (64, 2048, 4096)])
def test_silu_mul_linear(m, n, k):
    case("linear silu m=%d n=%d k=%d" % (m, n, k))
    rng = np.random.default_rng(m + n + k)
    gu = (rng.standard_normal((m, 2 * k)) * 2).astype(np.float16)
    w = workloads.weights(rng, (n, k))
    _check(gu, w, act="silu_mul")


def test_zero_rows_and_zero_row_output():
    rq = require_gpu()
    case("linear: M = 0 and an all-zero row")
    w_q, w_s = rq.quant_weights(dev(workloads.weights(np.random.default_rng(0), (32, 64))))
    y = rq.linear(torch.zeros((0, 64), dtype=torch.float16, device="cuda"), w_q, w_s)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)
    x = np.random.default_rng(1).standard_normal((3, 64)).astype(np.float16)
    x[1] = 0
    y = host(rq.linear(dev(x), w_q, w_s))
    assert np.all(y[1] == 0)


def test_dense_small_full():
    case("workload 1: dense 64 x 512 x 512")
    d = workloads.make(1)
    _check(d["x"], d["w"])


def test_merged_qkv_equals_split():
    rq = require_gpu()
    case("attention: merged QKV equals three linears")
    d = workloads.make(2, m=300, k=256)
    w_q, w_s = rq.quant_weights(dev(d["w_qkv"]))
    x = dev(d["x"])
    merged = host(rq.linear(x, w_q, w_s))
    parts = [host(rq.linear(x, w_q[i:i + 256].contiguous(), w_s[i:i + 256].contiguous())) for i in (0, 256, 512)]
    assert np.array_equal(merged, np.concatenate(parts, axis=1))


def _sample(m, rng, count=48):
    r = rng.choice(m, size=count, replace=False)
    return np.sort(np.concatenate([r, [0, m - 1]]))


@pytest.mark.slow
def test_attention_full_size():
    case("workload 2: attention 4096 tokens, QKV 6144 and O 2048")
    d = workloads.make(2)
    rng = np.random.default_rng(2)
    _check(d["x"], d["w_qkv"], sample_rows=_sample(4096, rng))
    _check(d["attn_out"], d["w_o"], sample_rows=_sample(4096, rng))


@pytest.mark.slow
def test_ffn_full_size_chain():
    rq = require_gpu()
    case("workload 3: FFN 4096 tokens, gate/up 16384, down 2048 over K = 8192")
    d = workloads.make(3)
    rng = np.random.default_rng(3)
    rows = _sample(4096, rng, 32)
    _check(d["x"], d["w_gu"], sample_rows=rows)
    # down projection over the GPU's own gate/up output
    wgu_q, wgu_s = rq.quant_weights(dev(d["w_gu"]))
    gu = rq.linear(dev(d["x"]), wgu_q, wgu_s)
    wdn_q, wdn_s = rq.quant_weights(dev(d["w_dn"]))
    y, dbg = rq.linear(gu, wdn_q, wdn_s, act="silu_mul", debug=True)
    gu_h, h, aq, a_s, y = host(gu), host(dbg["h"]), host(dbg["a_q"]), host(dbg["a_scale"]), host(y)
    assert ulp_diff16(h[rows], ffn.silu_mul(gu_h[rows], 8192)).max() <= 1
    hq, hs = quant.quantize_rows(h)
    assert np.array_equal(aq, hq) and np.array_equal(a_s.view(np.uint32), hs.view(np.uint32))
    ok, ratio, _ = linear.check(y[rows], hq[rows], hs[rows], host(wdn_q), host(wdn_s))
    assert ok, ratio


def test_determinism():
    rq = require_gpu()
    case("linear determinism 512 x 2048 x 2048")
    d = workloads.make(5, m=512, k=2048, f=64, f_moe=32, e=4)
    w_q, w_s = rq.quant_weights(dev(d["w_o"]))
    x = dev(d["x_o"])
    a = host(rq.linear(x, w_q, w_s))
    b = host(rq.linear(x, w_q, w_s))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128", "64x128", "64x256"])
@pytest.mark.parametrize("m,n,k", [(130, 272, 528), (257, 144, 192), (64, 512, 512), (300, 384, 2048)])
def test_every_tile_shape(monkeypatch, tile, m, n, k):
    case("linear tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
    monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(m + 3 * n + 7 * k)
    x = workloads.acts_channel_lognormal(rng, m, k)
    w = workloads.weights(rng, (n, k))
    _check(x, w)


@pytest.mark.parametrize("grid", ["3", "8"])
@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128", "64x128", "64x256"])
@pytest.mark.parametrize("m,n,k", [(300, 400, 1040), (130, 272, 208), (257, 144, 128), (70, 528, 64)])
def test_persistent_walk(monkeypatch, grid, tile, m, n, k):
    """Few workgroups, many tiles each: the LDS ring and the scale areas carried from one
    tile to the next (K of at least the ring depth), the per-tile restart (shorter K), odd
    slab counts and ragged K; 3 workgroups walk tiles in plain order, 8 in XCD slices."""
    case("linear walk grid=%s tile=%s m=%d n=%d k=%d" % (grid, tile, m, n, k))
    monkeypatch.setenv("RQ_GEMM_TILE", tile)
    monkeypatch.setenv("RQ_GEMM_GRID", grid)
    rng = np.random.default_rng(m * 3 + n + k)
    x = workloads.acts_student_t(rng, m, k)
    w = workloads.weights(rng, (n, k))
    _check(x, w)


@pytest.mark.parametrize("tile", [None, "256x256", "256x128", "128x128", "64x256"])
@pytest.mark.parametrize("m,f,k", [(130, 64, 272), (300, 320, 528), (64, 2048, 512)])
def test_gated_silu_output(monkeypatch, tile, m, f, k):
    """act='gate_silu' on interleaved gate/up weights writes exactly the h that the unfused
    path (plain gate/up linear, then the SiLU*up input transform of the down linear) makes."""
    rq = require_gpu()
    case("gated linear tile=%s m=%d f=%d k=%d" % (tile, m, f, k))
    if tile is not None:
        monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(m + f + k)
    x = workloads.acts_channel_lognormal(rng, m, k)
    w = workloads.weights(rng, (2 * f, k))
    wq, ws = rq.quant_weights(dev(w))
    order = torch.from_numpy(ffn.gate_up_order(f)).cuda()
    xd = dev(x)
    h = host(rq.linear(xd, wq[order].contiguous(), ws[order].contiguous(), act="gate_silu"))
    assert h.shape == (m, f)
    gu = rq.linear(xd, wq, ws)
    w_dn_q = torch.zeros((16, f), dtype=torch.uint8, device="cuda")
    _, dbg = rq.linear(gu, w_dn_q, torch.ones(16, device="cuda"), act="silu_mul", debug=True)
    assert np.array_equal(h.view(np.uint16), host(dbg["h"]).view(np.uint16))
    # and against the oracle's SiLU of the GPU's own gate/up output
    assert ulp_diff16(h, ffn.silu_mul(host(gu), f)).max() <= 1


def test_gated_needs_64_column_blocks():
    rq = require_gpu()
    case("gated linear: N % 64 != 0 is refused")
    wq = torch.zeros((96, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(rq.RqError):
        rq.linear(torch.zeros((4, 64), dtype=torch.float16, device="cuda"), wq,
                  torch.ones(96, device="cuda"), act="gate_silu")
