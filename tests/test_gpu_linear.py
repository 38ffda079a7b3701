"""GPU W8A8 linear vs the oracle.

Quantized activations (the bytes and scales the GEMM actually consumed, returned through
the debug outputs) must equal the oracle's bit for bit; FP16 outputs must lie within

    |y - y_ref| <= 2 ulp16(y_ref) + 1e-3 * s_x[m] * s_w[n] * sum_k |dec(x_q) dec(w_q)|

of the oracle's exactly accumulated result (``oracle.linear.check``).  Small shapes span
several 128-wide tiles with ragged M, N and K tails; the full-size workloads (dense 64 x
512 x 512, attention QKV/O at 4096 tokens, the FFN at 4096 tokens) are checked on every
quantized byte and every output row, in the launch configuration and (for the FFN) the
gated formulation the benchmark times.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import ffn, linear, quant
from tests import parity
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


@pytest.mark.slow
def test_attention_full_size():
    rq = require_gpu()
    d = workloads.make(2)
    # as the benchmark runs them: weights packed offline into the slab layout
    parity.linear_all_rows(rq, d["x"], d["w_qkv"], "workload 2: QKV 4096 x 6144 x 2048, every row", "slabs")
    parity.linear_all_rows(rq, d["attn_out"], d["w_o"], "workload 2: O 4096 x 2048 x 2048, every row", "slabs")


@pytest.mark.slow
def test_ffn_full_size_chain():
    """The dense FFN at 4096 tokens as the benchmark runs it (gated gate/up, down over
    K = 8192, slab-layout weights), every row, plus the unfused formulation bit for bit."""
    rq = require_gpu()
    d = workloads.make(3)
    parity.dense_ffn_gated(rq, d["x"], d["w_gu"], d["w_dn"], "workload 3: FFN 4096 tokens, F = 8192", "slabs")


def test_determinism():
    rq = require_gpu()
    case("linear determinism 512 x 2048 x 2048")
    d = workloads.make(5, m=512, k=2048, f=64, f_moe=32, e=4)
    w_q, w_s = rq.quant_weights(dev(d["w_o"]))
    x = dev(d["x_o"])
    a = host(rq.linear(x, w_q, w_s))
    b = host(rq.linear(x, w_q, w_s))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("tile", ["256x256", "256x192", "256x128", "128x128", "64x128", "64x256"])
@pytest.mark.parametrize("m,n,k", [(130, 272, 528), (257, 144, 192), (64, 512, 512), (300, 384, 2048)])
def test_every_tile_shape(monkeypatch, tile, m, n, k):
    case("linear tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
    monkeypatch.setenv("RQ_GEMM_TILE", tile)
    rng = np.random.default_rng(m + 3 * n + 7 * k)
    x = workloads.acts_channel_lognormal(rng, m, k)
    w = workloads.weights(rng, (n, k))
    _check(x, w)


@pytest.mark.parametrize("grid", ["3", "8"])
@pytest.mark.parametrize("tile", ["256x256", "256x192", "256x128", "128x128", "64x128", "64x256"])
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


@pytest.mark.parametrize("tile", [None, "256x256", "256x192", "256x128", "128x128", "64x256"])
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


def _splits(m, n, k):
    from fp8_quantized_generative_amd import _lib
    lib = _lib.load()
    extra = lib.rq_fp8_linear_workspace_size_ex(m, n, k, 0) - lib.rq_fp8_linear_workspace_size(m, k, 0)
    return (extra // 256 * 256) // (4 * m * n) if extra else 1


@pytest.mark.parametrize("m,n,k", [(512, 2048, 8192), (300, 6144, 4096), (64, 256, 4096), (1, 512, 8192),
                                   (1000, 1040, 4096)])
def test_split_k_small_m(m, n, k):
    """Few rows and a long K: the linear splits K into 2-8 parts whose FP32 sums a reduce kernel adds in
    order.  Every row within the oracle's tolerance; bit-identical on a second run; the
    unsplit call (smaller workspace) within the tolerance too."""
    rq = require_gpu()
    case("split-K linear m=%d n=%d k=%d" % (m, n, k))
    assert _splits(m, n, k) > 1
    rng = np.random.default_rng(m + n + k)
    x16, w16 = workloads.acts_student_t(rng, m, k), workloads.weights(rng, (n, k))
    ratio = _check(x16, w16)
    assert ratio <= 1
    wq, ws = rq.quant_weights(dev(w16))
    x = dev(x16)
    a, b = host(rq.linear(x, wq, ws)), host(rq.linear(x, wq, ws))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    plain = torch.empty(rq.linear_workspace_size(m, k), dtype=torch.uint8, device="cuda")
    y1 = host(rq.linear(x, wq, ws, workspace=plain))
    xq, xs = quant.quantize_rows(x16)
    ok, r1, _ = linear.check(y1, xq, xs, host(wq), host(ws))
    assert ok, r1


@pytest.mark.parametrize("m,f,k", [(512, 512, 4096), (96, 1024, 8192)])
def test_split_k_gated_equals_unfused(m, f, k):
    """The gated gate/up linear splits K exactly as the plain one (the part count depends on
    M, N and K only), so its h equals the unfused path's bit for bit."""
    rq = require_gpu()
    case("split-K gated m=%d f=%d k=%d" % (m, f, k))
    assert _splits(m, 2 * f, k) > 1
    rng = np.random.default_rng(m * f + k)
    x = dev(workloads.acts_channel_lognormal(rng, m, k))
    w = workloads.weights(rng, (2 * f, k))
    wq, ws = rq.quant_weights(dev(w))
    order = torch.from_numpy(ffn.gate_up_order(f)).cuda()
    h = host(rq.linear(x, wq[order].contiguous(), ws[order].contiguous(), act="gate_silu"))
    gu = rq.linear(x, wq, ws)
    _, dbg = rq.linear(gu, torch.zeros((16, f), dtype=torch.uint8, device="cuda"), torch.ones(16, device="cuda"),
                       act="silu_mul", debug=True)
    assert np.array_equal(h.view(np.uint16), host(dbg["h"]).view(np.uint16))
    assert ulp_diff16(h, ffn.silu_mul(host(gu), f)).max() <= 1
    # and the gate/up output itself against the oracle
    xq, xs = quant.quantize_rows(host(x))
    ok, r, _ = linear.check(host(gu), xq, xs, host(wq), host(ws))
    assert ok, r
