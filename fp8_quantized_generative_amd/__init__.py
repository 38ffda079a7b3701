"""MI355X (gfx950) W8A8 FP8 linear for OneRec-V2 post-training-quantized serving.

Python face of the C ABI in ``include/rq_fp8.h`` (``librq_fp8.so``).  Every step of the
computation runs in the library's HIP kernels; this module only marshals arguments.
PyTorch provides device memory and the current stream.

* ``quant_weights(w, wscale=...)``            offline E4M3 weight quantization (scales per
                                               output channel, per tensor or per 128x128 block)
* ``pack_weights(w_q)``                        offline repacking into the slab layout
                                               (``wlayout="slabs"`` in the linears)
* ``linear(x, w_q, w_scale, act=...)``         per-token quantization + FP8 GEMM + FP16 epilogue
* ``linear_noalloc(x, w_q, w_scale, out)``     the same without allocating (static device scratch)
* ``moe_grouped_linear(x, ids, w_q, w_scale, ...)``  routing plan + grouped GEMM (+ combine)
* ``attention_core(qkv, requests, length, heads)``  FP16 causal short-context attention (QKV -> O input)
* ``router_topk(x, w_gate, top_k)``            FP16 MoE gate logits -> top-k expert ids and weights
* ``topk(scores, k)``                          batched top-k of FP16 candidate rows (beam search)
* ``linear_workspace_size`` / ``moe_workspace_size``  scratch sizes for caller-held workspaces
"""

import contextlib
import ctypes

import torch

from . import _lib
from ._lib import (RQ_ACT_GATE_SILU, RQ_ACT_NONE, RQ_ACT_SILU_MUL, RQ_MOE_IN_PERMUTED, RQ_MOE_IN_TOKENS,  # noqa: F401
                   RQ_MOE_PLAN_READY,
                   RQ_MOE_OUT_COMBINED, RQ_MOE_OUT_PERMUTED, RQ_WSCALE_BLOCK128, RQ_WSCALE_CHANNEL,
                   RQ_WSCALE_TENSOR, RQ_WLAYOUT_SLABS, RQ_FP8_E4M3, RQ_FP8_E5M2, RQ_FLAG_EXPERT_ID, DebugOut,
                   RqError)

ACTS = {"none": RQ_ACT_NONE, "silu_mul": RQ_ACT_SILU_MUL, "gate_silu": RQ_ACT_GATE_SILU}
IN_LAYOUTS = {"tokens": RQ_MOE_IN_TOKENS, "permuted": RQ_MOE_IN_PERMUTED}
OUT_LAYOUTS = {"permuted": RQ_MOE_OUT_PERMUTED, "combined": RQ_MOE_OUT_COMBINED}
WSCALES = {"channel": RQ_WSCALE_CHANNEL, "tensor": RQ_WSCALE_TENSOR, "block128": RQ_WSCALE_BLOCK128}
AFMTS = {"e4m3": RQ_FP8_E4M3, "e5m2": RQ_FP8_E5M2}
WLAYOUTS = {"rows": 0, "slabs": RQ_WLAYOUT_SLABS}


def scale_shape(lead, n, k, wscale):
    """Shape of the FP32 weight scales of ``lead`` matrices [N, K] at granularity ``wscale``."""
    g = _code(WSCALES, wscale, "wscale")
    if g == RQ_WSCALE_TENSOR:
        return tuple(lead) if lead else (1,)
    if g == RQ_WSCALE_BLOCK128:
        return tuple(lead) + (n // 128, k // 128)
    return tuple(lead) + (n,)


def _code(table, v, what):
    if isinstance(v, str):
        if v not in table:
            raise ValueError("unknown %s %r" % (what, v))
        return table[v]
    return int(v)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise TypeError("%s must be contiguous" % name)
    return t


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %r, got %r" % (name, tuple(shape), tuple(t.shape)))


def _stream(t, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate on ``stream``: buffers this module allocates (outputs, workspaces, debug
    outputs) then belong to that stream in PyTorch's caching allocator, so a buffer freed
    while the stream's kernels still use it is only reused by later work on the same stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def quant_weights(w, w_q=None, w_scale=None, stream=None, wscale="channel"):
    """FP16 [N, K] or [B, N, K] -> (E4M3 bytes of the same shape, FP32 scales).

    Scales per ``wscale``: "channel" [N] / [B, N]; "tensor" [1] / [B]; "block128"
    [N/128, K/128] / [B, N/128, K/128]."""
    g = _code(WSCALES, wscale, "wscale")
    _dev(w, torch.float16, "w")
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N, K] or [B, N, K]")
    b, n, k = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    lead = tuple(w.shape[:-2])
    with _on(stream):
        if w_q is None:
            w_q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
        if w_scale is None:
            w_scale = torch.empty(scale_shape(lead, n, k, g), dtype=torch.float32, device=w.device)
    _dev(w_q, torch.uint8, "w_q")
    _dev(w_scale, torch.float32, "w_scale")
    _shape(w_q, w.shape, "w_q")
    _shape(w_scale, scale_shape(lead, n, k, g), "w_scale")
    st = _lib.load().rq_fp8_quant_weights_ex(_ptr(w), b, n, k, g, _ptr(w_q), _ptr(w_scale), _stream(w, stream))
    _lib.check("rq_fp8_quant_weights_ex", st)
    return w_q, w_scale


def pack_weights(w_q, out=None, stream=None):
    """E4M3 weights [N, K] or [B, N, K] (row layout) -> the same bytes in the slab layout
    [B, K/64, N, 64] (``rq_fp8_pack_weights``; K % 64 == 0), returned as a tensor of the input's
    shape that the linears take with ``wlayout="slabs"``."""
    _dev(w_q, torch.uint8, "w_q")
    if w_q.dim() not in (2, 3):
        raise ValueError("w_q must be [N, K] or [B, N, K]")
    b, n, k = (1,) + tuple(w_q.shape) if w_q.dim() == 2 else tuple(w_q.shape)
    with _on(stream):
        if out is None:
            out = torch.empty_like(w_q)
    _dev(out, torch.uint8, "out")
    _shape(out, w_q.shape, "out")
    st = _lib.load().rq_fp8_pack_weights(_ptr(w_q), b, n, k, _ptr(out), _stream(w_q, stream))
    _lib.check("rq_fp8_pack_weights", st)
    return out


def linear_workspace_size(m, k, act="none", n=None):
    """Workspace bytes of ``linear``; with ``n`` given, the size that also lets the call split
    K (small M, see ``rq_fp8_linear_workspace_size_ex``)."""
    a = _code(ACTS, act, "act")
    if n is None:
        return int(_lib.load().rq_fp8_linear_workspace_size(m, k, a))
    return int(_lib.load().rq_fp8_linear_workspace_size_ex(m, n, k, a))


def moe_workspace_size(t, top_k, e, n, k, in_layout="tokens", act="none", out_layout="permuted"):
    return int(_lib.load().rq_fp8_moe_workspace_size(
        t, top_k, e, n, k, _code(IN_LAYOUTS, in_layout, "in_layout"), _code(ACTS, act, "act"),
        _code(OUT_LAYOUTS, out_layout, "out_layout")))


def _debug(debug, q_rows, h_rows, k, act, device):
    if not debug:
        return None, None
    d = {"a_q": torch.empty((q_rows, k), dtype=torch.uint8, device=device),
         "a_scale": torch.empty((q_rows,), dtype=torch.float32, device=device),
         "h": torch.empty((h_rows, k), dtype=torch.float16, device=device) if act == RQ_ACT_SILU_MUL else None}
    s = DebugOut(d["a_q"].data_ptr(), d["a_scale"].data_ptr(), d["h"].data_ptr() if d["h"] is not None else 0)
    return d, s


def linear(x, w_q, w_scale, act="none", out=None, workspace=None, debug=False, stream=None, wscale="channel",
           afmt="e4m3", wlayout="rows"):
    """W8A8 FP8 linear: FP16 x [M, K] (or [M, 2K] for ``act='silu_mul'``) -> FP16 y [M, N]
    (or h [M, N/2] for ``act='gate_silu'``, whose weight rows interleave 32 gate and 32 up
    features; see ``interleave_gate_up``).

    With ``debug=True`` returns ``(y, {"a_q", "a_scale", "h"})``: the quantized GEMM input
    (and the SiLU*up rows).  ``wscale`` names the granularity of ``w_scale`` (see
    ``quant_weights``); ``afmt`` the format the activations are quantized to ("e4m3" or
    "e5m2"); ``wlayout`` the byte layout of ``w_q`` ("rows", or "slabs" from ``pack_weights``).
    """
    a = _code(ACTS, act, "act")
    g = _code(WSCALES, wscale, "wscale")
    wl = _code(WLAYOUTS, wlayout, "wlayout")
    f = _code(AFMTS, afmt, "afmt")
    _dev(x, torch.float16, "x")
    _dev(w_q, torch.uint8, "w_q")
    _dev(w_scale, torch.float32, "w_scale")
    if x.dim() != 2 or w_q.dim() != 2:
        raise ValueError("x and w_q must be 2-D")
    m = x.shape[0]
    n, k = w_q.shape
    if x.shape[1] != (2 * k if a == RQ_ACT_SILU_MUL else k):
        raise ValueError("x width %d does not match K=%d for act=%r" % (x.shape[1], k, act))
    n_out = n // 2 if a == RQ_ACT_GATE_SILU else n
    lib = _lib.load()
    with _on(stream):
        if out is None:
            out = torch.empty((m, n_out), dtype=torch.float16, device=x.device)
        ws = _workspace(lib.rq_fp8_linear_workspace_size_ex(m, n, k, a), x.device, workspace)
        dbg, dbg_s = _debug(debug, m, m, k, a, x.device)
    _dev(out, torch.float16, "out")
    _shape(out, (m, n_out), "out")
    _shape(w_scale, scale_shape((), n, k, g), "w_scale")
    st = lib.rq_fp8_linear_ex(_ptr(x), m, k, a, f, _ptr(w_q), _ptr(w_scale), g | wl, n, _ptr(out), _ptr(ws),
                              ws.numel(), ctypes.byref(dbg_s) if dbg_s is not None else None,
                              _stream(x, stream))
    _lib.check("rq_fp8_linear_ex", st)
    return (out, dbg) if debug else out


def linear_noalloc(x, w_q, w_scale, out, act="none", stream=None):
    """``linear`` without any allocation: the caller passes ``out`` (FP16 [M, N], or
    [M, N/2] for ``act='gate_silu'``) and the quantized activations live in the library's
    static device buffer (``RQ_STATIC_SCRATCH_BYTES`` per GPU; calls that overlap on one GPU
    race on it).  E4M3 activations, per-channel weight scales."""
    a = _code(ACTS, act, "act")
    _dev(x, torch.float16, "x")
    _dev(w_q, torch.uint8, "w_q")
    _dev(w_scale, torch.float32, "w_scale")
    _dev(out, torch.float16, "out")
    if x.dim() != 2 or w_q.dim() != 2:
        raise ValueError("x and w_q must be 2-D")
    m = x.shape[0]
    n, k = w_q.shape
    if x.shape[1] != (2 * k if a == RQ_ACT_SILU_MUL else k):
        raise ValueError("x width %d does not match K=%d for act=%r" % (x.shape[1], k, act))
    _shape(out, (m, n // 2 if a == RQ_ACT_GATE_SILU else n), "out")
    _shape(w_scale, (n,), "w_scale")
    st = _lib.load().rq_fp8_linear_noalloc(_ptr(x), m, k, a, _ptr(w_q), _ptr(w_scale), n, _ptr(out),
                                           _stream(x, stream))
    _lib.check("rq_fp8_linear_noalloc", st)
    return out


def moe_grouped_linear(x, topk_ids, w_q, w_scale, in_layout="tokens", act="none",
                       out_layout="permuted", topk_w=None, out=None, workspace=None,
                       debug=False, stream=None, wscale="channel", afmt="e4m3", plan_ready=False,
                       wlayout="rows"):
    """Expert grouped W8A8 linear.

    ``x``: FP16 [T, K*] (tokens) or [T*top_k, K*] (permuted), K* = 2K for ``silu_mul``;
    ``topk_ids``: int32 [T, top_k]; ``w_q``: uint8 [E, N, K]; ``w_scale``: FP32 [E, N] (or the
    ``wscale`` layout with E matrices, see ``quant_weights``);
    ``topk_w``: FP16 [T, top_k] for ``out_layout='combined'``.
    ``plan_ready``: the ``workspace`` given already holds the routing plan of these ``topk_ids``
    from an earlier call (permuted input only; see ``RQ_MOE_PLAN_READY``).
    ``wlayout``: byte layout of ``w_q`` ("rows", or "slabs" from ``pack_weights``).
    Returns FP16 [T*top_k, N] (permuted) or [T, N] (combined), plus the debug dict when
    ``debug=True``: ``a_q`` / ``a_scale`` hold the GEMM operand, one row per routed slot in
    the permuted order; ``h`` (``silu_mul``) one row per input row.
    """
    il = _code(IN_LAYOUTS, in_layout, "in_layout")
    a = _code(ACTS, act, "act")
    ol = _code(OUT_LAYOUTS, out_layout, "out_layout")
    g = _code(WSCALES, wscale, "wscale")
    wl = _code(WLAYOUTS, wlayout, "wlayout")
    f = _code(AFMTS, afmt, "afmt")
    _dev(x, torch.float16, "x")
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(w_q, torch.uint8, "w_q")
    _dev(w_scale, torch.float32, "w_scale")
    if topk_w is not None:
        _dev(topk_w, torch.float16, "topk_w")
    t, top_k = topk_ids.shape
    e, n, k = w_q.shape
    r = t * top_k
    rows = t if il == RQ_MOE_IN_TOKENS else r
    if tuple(x.shape) != (rows, 2 * k if a == RQ_ACT_SILU_MUL else k):
        raise ValueError("x shape %r does not match the layout" % (tuple(x.shape),))
    out_shape = (t if ol == RQ_MOE_OUT_COMBINED else r, n // 2 if a == RQ_ACT_GATE_SILU else n)
    lib = _lib.load()
    with _on(stream):
        if out is None:
            out = torch.empty(out_shape, dtype=torch.float16, device=x.device)
        ws = _workspace(lib.rq_fp8_moe_workspace_size(t, top_k, e, n, k, il, a, ol), x.device, workspace)
        dbg, dbg_s = _debug(debug, r, rows, k, a, x.device)
    _dev(out, torch.float16, "out")
    _shape(out, out_shape, "out")
    _shape(w_scale, scale_shape((e,), n, k, g), "w_scale")
    if plan_ready and workspace is None:
        raise ValueError("plan_ready needs the workspace that holds the plan")
    st = lib.rq_fp8_moe_grouped_linear_ex(
        _ptr(x), il | (RQ_MOE_PLAN_READY if plan_ready else 0), a, f, _ptr(topk_ids), _ptr(topk_w), t, top_k,
        _ptr(w_q), _ptr(w_scale), g | wl, e, n, k,
        _ptr(out), ol, _ptr(ws), ws.numel(), ctypes.byref(dbg_s) if dbg_s is not None else None,
        _stream(x, stream))
    _lib.check("rq_fp8_moe_grouped_linear_ex", st)
    return (out, dbg) if debug else out


def router_topk(x, w_gate, top_k=2, topk_ids=None, topk_w=None, logits=False, stream=None):
    """FP16 MoE gate: x [T, K] FP16 and gate weights [E, K] FP16 -> (topk_ids int32 [T, top_k],
    topk_w FP16 [T, top_k]) - the routing inputs of ``moe_grouped_linear`` - plus the FP32
    logits [T, E] when ``logits=True``."""
    _dev(x, torch.float16, "x")
    _dev(w_gate, torch.float16, "w_gate")
    if x.dim() != 2 or w_gate.dim() != 2 or x.shape[1] != w_gate.shape[1]:
        raise ValueError("x [T, K] and w_gate [E, K] must share K")
    t, k = x.shape
    e = w_gate.shape[0]
    with _on(stream):
        if topk_ids is None:
            topk_ids = torch.empty((t, top_k), dtype=torch.int32, device=x.device)
        if topk_w is None:
            topk_w = torch.empty((t, top_k), dtype=torch.float16, device=x.device)
        lg = torch.empty((t, e), dtype=torch.float32, device=x.device) if logits else None
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float16, "topk_w")
    _shape(topk_ids, (t, top_k), "topk_ids")
    _shape(topk_w, (t, top_k), "topk_w")
    st = _lib.load().rq_moe_router_topk(_ptr(x), t, k, _ptr(w_gate), e, top_k, _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(lg), _stream(x, stream))
    _lib.check("rq_moe_router_topk", st)
    return (topk_ids, topk_w, lg) if logits else (topk_ids, topk_w)


def attention_core(qkv, requests, length, heads, head_dim=128, out=None, stream=None):
    """Causal short-context attention over the merged QKV output: qkv FP16
    [requests * length, 3 * heads * head_dim] -> FP16 [requests * length, heads * head_dim]."""
    _dev(qkv, torch.float16, "qkv")
    hidden = heads * head_dim
    _shape(qkv, (requests * length, 3 * hidden), "qkv")
    if out is None:
        with _on(stream):
            out = torch.empty((requests * length, hidden), dtype=torch.float16, device=qkv.device)
    _dev(out, torch.float16, "out")
    _shape(out, (requests * length, hidden), "out")
    st = _lib.load().rq_attention_core(_ptr(qkv), requests, length, heads, head_dim, _ptr(out), _stream(qkv, stream))
    _lib.check("rq_attention_core", st)
    return out


def topk_workspace_size(rows, n, k):
    return int(_lib.load().rq_topk_workspace_size(rows, n, k))


def topk(scores, k, idx=None, vals=None, workspace=None, stream=None):
    """Batched top-k of FP16 rows [rows, n]: ``(idx int32 [rows, k], vals FP16 [rows, k])``,
    ranked by score (larger first, -0 below +0), equal scores by lower index."""
    _dev(scores, torch.float16, "scores")
    if scores.dim() != 2:
        raise ValueError("scores must be [rows, n]")
    rows, n = scores.shape
    lib = _lib.load()
    with _on(stream):
        if idx is None:
            idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
        if vals is None:
            vals = torch.empty((rows, k), dtype=torch.float16, device=scores.device)
        need = lib.rq_topk_workspace_size(rows, n, k) if 1 <= k <= n else 0
        ws = _workspace(need, scores.device, workspace)
    _dev(idx, torch.int32, "idx")
    _dev(vals, torch.float16, "vals")
    _shape(idx, (rows, k), "idx")
    _shape(vals, (rows, k), "vals")
    st = lib.rq_topk(_ptr(scores), rows, n, k, _ptr(idx), _ptr(vals), _ptr(ws), ws.numel(), _stream(scores, stream))
    _lib.check("rq_topk", st)
    return idx, vals


def debug_flag(clear=False):
    """The current device's error word (waits for all work on the device): bit
    ``RQ_FLAG_EXPERT_ID`` is set once a routing id outside [0, E) reached
    ``moe_grouped_linear``.  ``clear=True`` resets it."""
    v = _lib.load().rq_debug_flag(1 if clear else 0)
    if v < 0:
        raise RqError("rq_debug_flag", _lib.RQ_ERR_HIP)
    return v


def interleave_gate_up(w_gu, block=32):
    """Reorder gate/up weight rows [gate (F) | up (F)] (any leading expert dims) into blocks of
    `block` alternating gate and up rows, the layout ``act='gate_silu'`` expects.  Offline
    weight preparation; works on any tensor (or array) with rows on the second-to-last axis
    (FP16 weights before quantization, or E4M3 bytes with their scales as [..., 2F, 1])."""
    f2 = w_gu.shape[-2]
    if f2 % (2 * block) != 0:
        raise ValueError("gate/up rows (%d) must be a multiple of %d" % (f2, 2 * block))
    f = f2 // 2
    lead = tuple(w_gu.shape[:-2])
    g = w_gu[..., :f, :].reshape(lead + (f // block, 1, block, w_gu.shape[-1]))
    u = w_gu[..., f:, :].reshape(lead + (f // block, 1, block, w_gu.shape[-1]))
    cat = torch.cat if isinstance(w_gu, torch.Tensor) else __import__("numpy").concatenate
    return cat([g, u], -3).reshape(w_gu.shape)
