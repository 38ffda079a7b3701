#!/usr/bin/env python3
"""Throughput of the W8A8 FP8 linear hot path on one MI355X (gfx950).

A step is one pass of the whole path over one batch of each synthetic workload, at full
size, with inputs and quantized weights resident in HBM:

* attention projections: 4096 tokens x hidden 2048, merged QKV (N = 6144) and O (2048);
* dense FFN: 4096 tokens, gate/up (N = 16384) writing h = SiLU(g)*up from its epilogue
  (gate/up weight rows interleaved offline), h re-quantization, down (K = 8192);
* sparse MoE: 16384 tokens, top-2 of 32 Zipf-loaded experts, grouped gate/up (8192) writing
  h, grouped down (K = 4096) and the weighted combine;
* small-M layer: 512 rows through QKV, O, the dense FFN and the MoE expert FFN.

Each linear runs per-token activation quantization, the FP8 MFMA GEMM with FP32
accumulation and the fused dequantization to FP16 (weights are quantized once, offline,
before timing).  ``value`` is algorithmic FP8 TFLOP/s: sum of 2*M*N*K over the real rows
of every GEMM in the step (MoE counted over routed rows, no padding), divided by the
wall time of K steps bracketed by device synchronizations.

Also reported: the roofline of the dominant kernel (the MoE gate/up grouped GEMM),
timed with HIP events around that launch inside every timed step; per-kernel event
timings after the timed region; and the CPU oracle timed on a bounded sample.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=50,
                    help="repetitions of each isolated, cache-flushed kernel timing after the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel breakdown")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the variants (per-tensor FFN and 128x128-block MoE weight scales, E5M2 activations)")
    ap.add_argument("--rocprof-summary", default=None, metavar="PATH",
                    help="print per-(kernel, grid) dispatch statistics of a rocprofv3 output "
                         "(a *_results.db, a *_kernel_trace.csv, or a directory holding one) and exit")
    ap.add_argument("--kernel-stats", default=None, metavar="PATH",
                    help="print this library's kernels from a rocprofv3 --stats output (*_kernel_stats.csv, or a "
                         "directory holding one): calls and average duration per kernel instantiation, and exit")
    ap.add_argument("--wlayout", default="slabs", choices=["slabs", "rows"],
                    help="byte layout of the quantized weights, chosen offline: the slab layout of "
                         "rq_fp8_pack_weights (default) or the plain [N][K] rows")
    ap.add_argument("--only", default=None,
                    help="comma list of attention,ffn,moe,layer_small_m to restrict the step (profiling)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0, metavar="MB",
                    help="after the timed steps, one device-to-device copy of MB MiB (the known-size kernel "
                         "that scales HBM byte counters)")
    ap.add_argument("--traffic-summary", nargs=3, default=None, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a bench command with "
                         "--calibrate-copy-mb, write the dominant kernel's HBM traffic per launch to OUT (json)")
    ap.add_argument("--pmc-summary", default=None, metavar="PATH",
                    help="print FP8 MFMA counts, MFMA busy fraction and clock per GEMM call from a rocprofv3 "
                         "--pmc database (SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_F8 SQ_VALU_MFMA_BUSY_CYCLES "
                         "SQ_INSTS_VALU GRBM_GUI_ACTIVE) and exit")
    ap.add_argument("--pmc-dump", nargs="+", default=None, metavar="PATH",
                    help="print every counter of rocprofv3 --pmc databases per GEMM call of the step and exit")
    ap.add_argument("--steps-in-profile", type=int, default=None,
                    help="with --rocprof-summary / --traffic-summary: steps (warmup + timed) the profiled "
                         "command ran")
    return ap.parse_args()


# Calls of one step, in launch order: (workload, call, kind), and the kernels each kind
# launches (the library's choices at these shapes).  "linear": the row quantizer and the GEMM;
# "linear_split" (512 x 2048 x 8192: K cut in 4 parts): also the reduce kernel that adds the
# parts; "moe": the single-workgroup routing plan (up to 8192 slots), the quantizer and the
# grouped GEMM; "moe_large" (32768 slots): the three plan kernels instead; "moe_combined" (the
# down call, which reuses the gate/up call's plan): the quantizer, the grouped GEMM and the
# weighted combine.
STEP = [
    ("attention", "qkv", "linear"), ("attention", "o", "linear"),
    ("ffn", "gate_up", "linear"), ("ffn", "down", "linear"),
    ("moe", "gate_up", "moe_large"), ("moe", "down", "moe_combined"),
    ("layer_small_m", "qkv", "linear"), ("layer_small_m", "o", "linear"),
    ("layer_small_m", "gate_up", "linear"), ("layer_small_m", "down", "linear_split"),
    ("layer_small_m", "moe_gate_up", "moe"), ("layer_small_m", "moe_down", "moe_combined"),
]
DOMINANT = ("moe", "gate_up")
KERNELS = {"linear": ["quant", "gemm"], "linear_split": ["quant", "gemm", "reduce"],
           "moe": ["plan", "quant", "gemm"], "moe_large": ["plan_hist", "plan_scan", "plan_scatter", "quant", "gemm"],
           "moe_combined": ["quant", "gemm", "combine"]}
OUR_KERNELS = ("quant_rows", "gemm_fp8_kernel", "splitk_reduce", "plan_single", "plan_hist", "plan_scan",
               "plan_scatter", "combine_kernel")


def step_dispatches(only):
    """(label, kind) of every kernel one step launches, in order."""
    want = set(only.split(",")) if only else {w for w, _, _ in STEP}
    return [("%s %s" % (w, c), k) for w, c, kind in STEP if w in want for k in KERNELS[kind]]


def stats_us(ms_list):
    """Median, 10th and 90th percentile and mean of durations given in ms, in us."""
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2), "n": int(a.size)}


class Flush:
    """Evicts L2 and the 256 MB last-level cache before each isolated repetition, so that
    HBM-bound timings cannot be served from cache: a read of 1 GiB of scratch (a sum on the
    current stream).  Reading, not writing, leaves the caches full of clean lines, so the
    timed kernel does not pay for writing the flush's dirty lines back to HBM."""

    def __init__(self, torch, mib=1024):
        self.torch = torch
        self.buf = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        self.out = torch.zeros((), dtype=torch.float32, device="cuda")
        self.mib = mib

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.out)


class Hip:
    """The HIP runtime already loaded by torch: events for kernel-level timing."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ev, ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


class Path:
    """Device-resident inputs, quantized weights, outputs and workspaces of one step."""

    def __init__(self, rq, torch, only=None, variants=True, wlayout="slabs"):
        import workloads
        self.rq, self.torch = rq, torch
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        self.calls = []     # (workload, label, kind, flops, bytes_moved, fn)
        self.qbytes = []    # per call: bytes the row quantizer must move
        # variants, timed apart from the step: (workload, call, variant, flops, index of the
        # per-channel E4M3 call of the same shape, fn)
        self.variants = []
        self.router = None  # (bytes per launch, fn) of the MoE router, timed apart from the step
        self.attention = None  # the same for the attention core
        self.beam = []         # (label, bytes per call, fn, torch.topk of the same rows) of the beam top-k workloads
        self.flops = 0
        want = set(only.split(",")) if only else {"attention", "ffn", "moe", "layer_small_m"}

        self.wlayout = wlayout

        def qw(w16, wscale="channel"):
            # offline (untimed): quantize, then repack into the layout the step uses
            wq, ws = rq.quant_weights(dev(w16), wscale=wscale)
            if wlayout == "slabs":
                wq = rq.pack_weights(wq)
            return wq, ws

        def ffn_workspace(t, e, f, k):
            # one workspace for both calls of an expert FFN: the down call reuses the routing plan
            # the gate/up call left at its front
            size = max(rq.moe_workspace_size(t, 2, e, 2 * f, k, "tokens", "gate_silu", "permuted"),
                       rq.moe_workspace_size(t, 2, e, k, f, "permuted", "none", "combined"))
            return torch.empty(size, dtype=torch.uint8, device="cuda")

        def qw_gated(w16):
            # gate/up rows interleaved in blocks of 32 (offline, untimed): the gate/up GEMM
            # then writes h = silu(g) * u directly
            return qw(rq.interleave_gate_up(w16))

        def add_linear(work, label, x, wq, ws, act="none"):
            m = x.shape[0]
            n, k = wq.shape
            out = torch.empty((m, n // 2 if act == "gate_silu" else n), dtype=torch.float16, device="cuda")
            ws_t = torch.empty(max(rq.linear_workspace_size(m, k, act, n=n), 1), dtype=torch.uint8, device="cuda")
            fl = 2 * m * n * k
            # bytes that must cross HBM at least once: activations in, weights, output
            by = x.numel() * 2 + wq.numel() + out.numel() * 2
            self.calls.append((work, label, "linear", fl, by,
                               lambda: rq.linear(x, wq, ws, act=act, out=out, workspace=ws_t, wlayout=wlayout)))
            # the row quantizer: FP16 rows in, E4M3 rows and FP32 scales out
            self.qbytes.append(x.numel() * 2 + m * k + 4 * m)
            self.flops += fl
            return out

        def add_moe(work, label, x, ids, wq, ws, il, act, ol, topk_w=None, ws_t=None, plan_ready=False):
            t, top_k = ids.shape
            e, n, k = wq.shape
            r = t * top_k
            n_out = n // 2 if act == "gate_silu" else n
            out = torch.empty((t if ol == "combined" else r, n_out), dtype=torch.float16, device="cuda")
            if ws_t is None:
                ws_t = torch.empty(rq.moe_workspace_size(t, top_k, e, n, k, il, act, ol), dtype=torch.uint8,
                                   device="cuda")
            fl = 2 * r * n * k
            touched = int(torch.unique(ids).numel())  # experts with rows: only their weights are read
            by = x.numel() * 2 + touched * n * k + (t if ol == "combined" else r) * n_out * 2
            self.calls.append((work, label, "moe", fl, by,
                               lambda: rq.moe_grouped_linear(x, ids, wq, ws, il, act, ol, topk_w=topk_w,
                                                             out=out, workspace=ws_t, plan_ready=plan_ready,
                                                             wlayout=wlayout)))
            # the row quantizer reads each input row once and writes one E4M3 row and scale per
            # routed slot
            self.qbytes.append(x.numel() * 2 + r * k + 4 * r)
            self.flops += fl
            return out

        # the small dense linear (64 x 512 x 512), timed on its own after the timed steps: its
        # time is launch latency, so it is reported in microseconds and kept out of the step
        d1 = workloads.make(1)
        w1 = qw(d1["w"])
        x1 = dev(d1["x"])
        y1 = torch.empty((64, 512), dtype=torch.float16, device="cuda")
        ws1 = torch.empty(rq.linear_workspace_size(64, 512, n=512), dtype=torch.uint8, device="cuda")
        self.c1 = (2 * 64 * 512 * 512, lambda: rq.linear(x1, *w1, out=y1, workspace=ws1, wlayout=wlayout))
        if variants:
            # beam top-k: 32 requests x (16 beams | 512 beams) x 512 codes, keep 16 | 512
            for beams, keep in ((16, 16), (512, 512)):
                sc = dev(workloads.beam_scores(np.random.default_rng(3000 + beams), 32, beams, 512))
                n = beams * 512
                ti = torch.empty((32, keep), dtype=torch.int32, device="cuda")
                tv = torch.empty((32, keep), dtype=torch.float16, device="cuda")
                tw = torch.empty(max(rq.topk_workspace_size(32, n, keep), 1), dtype=torch.uint8, device="cuda")
                self.beam.append(("32 requests x %d beams x 512 codes, keep %d" % (beams, keep),
                                  32 * n * 2 + 32 * keep * 6,
                                  lambda sc=sc, keep=keep, ti=ti, tv=tv, tw=tw: rq.topk(sc, keep, idx=ti, vals=tv,
                                                                                       workspace=tw),
                                  lambda sc=sc, keep=keep: torch.topk(sc, keep, dim=1)))
        self.config = {}
        if "attention" in want:
            d = workloads.make(2)
            wqkv = qw(d["w_qkv"])
            wo = qw(d["w_o"])
            qkv = add_linear("attention", "qkv", dev(d["x"]), *wqkv)
            add_linear("attention", "o", dev(d["attn_out"]), *wo)
            if variants:
                # the FP16 attention core between them, on the QKV call's output (128 requests x
                # 32 positions, 16 heads of 128)
                ao = torch.empty((4096, 2048), dtype=torch.float16, device="cuda")
                self.attention = (qkv.numel() * 2 + ao.numel() * 2,
                                  lambda qkv=qkv, ao=ao: rq.attention_core(qkv, 128, 32, 16, out=ao))
            self.config["attention"] = "4096 tokens x 2048; QKV 6144, O 2048"
        if "ffn" in want:
            d = workloads.make(3)
            wgu, wdn = qw_gated(d["w_gu"]), qw(d["w_dn"])
            h = add_linear("ffn", "gate_up", dev(d["x"]), *wgu, act="gate_silu")
            add_linear("ffn", "down", h, *wdn)
            if variants:
                # the dense FFN with one scale per weight tensor
                x3 = dev(d["x"])
                tgu = qw(rq.interleave_gate_up(d["w_gu"]), wscale="tensor")
                tdn = qw(d["w_dn"], wscale="tensor")
                h_t = torch.empty_like(h)
                y_t = torch.empty((4096, 2048), dtype=torch.float16, device="cuda")
                ws_gu = torch.empty(rq.linear_workspace_size(4096, 2048), dtype=torch.uint8, device="cuda")
                ws_dn = torch.empty(rq.linear_workspace_size(4096, 8192), dtype=torch.uint8, device="cuda")
                n0 = len(self.calls)
                self.variants.append(("ffn", "gate_up", "tensor", self.calls[n0 - 2][3], n0 - 2,
                                      lambda x3=x3, tgu=tgu, h_t=h_t, ws_gu=ws_gu: rq.linear(
                                          x3, *tgu, act="gate_silu", out=h_t, workspace=ws_gu, wscale="tensor",
                                          wlayout=wlayout)))
                self.variants.append(("ffn", "down", "tensor", self.calls[n0 - 1][3], n0 - 1,
                                      lambda h_t=h_t, tdn=tdn, y_t=y_t, ws_dn=ws_dn: rq.linear(
                                          h_t, *tdn, out=y_t, workspace=ws_dn, wscale="tensor", wlayout=wlayout)))
                # the dense FFN with E5M2 activations (per-channel E4M3 weights)
                self.variants.append(("ffn", "gate_up", "e5m2 activations", self.calls[n0 - 2][3], n0 - 2,
                                      lambda x3=x3, w=wgu, h_t=h_t, ws_gu=ws_gu: rq.linear(
                                          x3, *w, act="gate_silu", out=h_t, workspace=ws_gu, afmt="e5m2",
                                          wlayout=wlayout)))
                self.variants.append(("ffn", "down", "e5m2 activations", self.calls[n0 - 1][3], n0 - 1,
                                      lambda h_t=h_t, w=wdn, y_t=y_t, ws_dn=ws_dn: rq.linear(
                                          h_t, *w, out=y_t, workspace=ws_dn, afmt="e5m2", wlayout=wlayout)))
            self.config["ffn"] = "4096 tokens x 2048; gate/up 2x8192, down K=8192"
        if "moe" in want:
            d = workloads.make(4)
            wgu, wdn = qw_gated(d["w_gu"]), qw(d["w_dn"])
            ids, tw = dev(d["ids"].astype(np.int32)), dev(d["topk_w"])
            counts = np.bincount(d["ids"].reshape(-1), minlength=32)
            shared = ffn_workspace(16384, 32, 4096, 2048)
            h = add_moe("moe", "gate_up", dev(d["x"]), ids, *wgu, "tokens", "gate_silu", "permuted", ws_t=shared)
            self.dominant = len(self.calls) - 1
            add_moe("moe", "down", h, ids, *wdn, "permuted", "none", "combined", topk_w=tw, ws_t=shared,
                    plan_ready=True)
            if variants:
                # expert weights with one scale per 128 x 128 block
                x4 = dev(d["x"])
                bgu = qw(rq.interleave_gate_up(d["w_gu"]), wscale="block128")
                bdn = qw(d["w_dn"], wscale="block128")
                h_b = torch.empty_like(h)
                y_b = torch.empty((16384, 2048), dtype=torch.float16, device="cuda")
                ws_gu = torch.empty(rq.moe_workspace_size(16384, 2, 32, 8192, 2048, "tokens", "gate_silu", "permuted"),
                                    dtype=torch.uint8, device="cuda")
                ws_dn = torch.empty(rq.moe_workspace_size(16384, 2, 32, 2048, 4096, "permuted", "none", "combined"),
                                    dtype=torch.uint8, device="cuda")
                # the FP16 router that would produce this step's routing (synthetic gate weights)
                wg = dev((np.random.default_rng(1104).standard_normal((32, 2048)) / np.sqrt(2048)).astype(np.float16))
                r_ids = torch.empty((16384, 2), dtype=torch.int32, device="cuda")
                r_w = torch.empty((16384, 2), dtype=torch.float16, device="cuda")
                self.router = (16384 * 2048 * 2 + 32 * 2048 * 2 + 16384 * 2 * 6,
                               lambda x4=x4, wg=wg, r_ids=r_ids, r_w=r_w: rq.router_topk(
                                   x4, wg, 2, topk_ids=r_ids, topk_w=r_w))
                n0 = len(self.calls)
                self.variants.append(("moe", "gate_up", "block128", self.calls[n0 - 2][3], n0 - 2,
                                      lambda x4=x4, ids=ids, bgu=bgu, h_b=h_b, ws_gu=ws_gu: rq.moe_grouped_linear(
                                          x4, ids, *bgu, "tokens", "gate_silu", "permuted", out=h_b, workspace=ws_gu,
                                          wscale="block128", wlayout=wlayout)))
                self.variants.append(("moe", "down", "block128", self.calls[n0 - 1][3], n0 - 1,
                                      lambda h_b=h_b, ids=ids, bdn=bdn, tw=tw, y_b=y_b, ws_dn=ws_dn:
                                      rq.moe_grouped_linear(h_b, ids, *bdn, "permuted", "none", "combined", topk_w=tw,
                                                            out=y_b, workspace=ws_dn, wscale="block128",
                                                            wlayout=wlayout)))
            self.config["moe"] = ("16384 tokens x 2048; top-2 of 32 experts (Zipf 1.1; max %d, min nonzero %d, "
                                  "%d empty experts; 32768 routed rows); gate/up 2x4096, down K=4096"
                                  % (counts.max(), counts[counts > 0].min(), int((counts == 0).sum())))
            del d
        if "layer_small_m" in want:
            d = workloads.make(5)
            add_linear("layer_small_m", "qkv", dev(d["x_qkv"]), *qw(d["w_qkv"]))
            add_linear("layer_small_m", "o", dev(d["x_o"]), *qw(d["w_o"]))
            h = add_linear("layer_small_m", "gate_up", dev(d["x_ffn"]), *qw_gated(d["w_gu"]), act="gate_silu")
            add_linear("layer_small_m", "down", h, *qw(d["w_dn"]))
            ids, tw = dev(d["ids"].astype(np.int32)), dev(d["topk_w"])
            shared5 = ffn_workspace(512, 32, 4096, 2048)
            h2 = add_moe("layer_small_m", "moe_gate_up", dev(d["x_moe"]), ids, *qw_gated(d["w_gu_moe"]),
                         "tokens", "gate_silu", "permuted", ws_t=shared5)
            add_moe("layer_small_m", "moe_down", h2, ids, *qw(d["w_dn_moe"]), "permuted", "none",
                    "combined", topk_w=tw, ws_t=shared5, plan_ready=True)
            self.config["layer_small_m"] = "512 rows (32 requests x 16 beams); one layer: QKV, O, FFN 8192, MoE 4096"
            del d
        if not hasattr(self, "dominant"):
            self.dominant = max(range(len(self.calls)), key=lambda i: self.calls[i][3])
        self.quant_dominant = max(range(len(self.calls)), key=lambda i: self.qbytes[i])
        torch.cuda.synchronize()

    def step(self, hooks=()):
        for i, c in enumerate(self.calls):
            for h in hooks:
                if i == h[0]:
                    self.rq._lib.load().rq_time_next_kernel(h[1], h[2], h[3])
            c[5]()


class KernelTimer:
    """Times one kernel kind of a library call with HIP events (``rq_time_next_kernel``), or a
    whole sequence of calls, on the current stream; ``flush`` runs before every repetition."""

    def __init__(self, hip, torch, flush):
        from fp8_quantized_generative_amd import _lib
        self.hip, self.torch, self.flush, self.lib = hip, torch, flush, _lib.load()
        self.a, self.b = hip.event(), hip.event()

    def kernel(self, fn, kind, reps):
        fn()  # first call outside the timing (code objects, allocator)
        ts = []
        for _ in range(reps):
            if self.flush is not None:
                self.flush()
            self.lib.rq_time_next_kernel(kind, self.a, self.b)
            fn()
            ts.append(self.hip.elapsed_ms(self.a, self.b))
        return ts

    def sequence(self, fns, reps):
        for fn in fns:
            fn()
        ts = []
        for _ in range(reps):
            if self.flush is not None:
                self.flush()
            stream = self.torch.cuda.current_stream().cuda_stream
            self.hip.record(self.a, stream)
            for fn in fns:
                fn()
            self.hip.record(self.b, stream)
            ts.append(self.hip.elapsed_ms(self.a, self.b))
        return ts


def kernel_breakdown(path, timer, reps):
    """Per call: the GEMM and the row quantizer, each timed in isolation with L2 and the
    last-level cache flushed before every repetition (HBM-cold weights and inputs; the GEMM's
    activation operand was just written by the call's own quantizer)."""
    from fp8_quantized_generative_amd import _lib
    rows = []
    for i, (work, label, kind, fl, by, fn) in enumerate(path.calls):
        g = stats_us(timer.kernel(fn, _lib.RQ_KERNEL_GEMM, reps))
        q = stats_us(timer.kernel(fn, _lib.RQ_KERNEL_QUANT, reps))
        qgbs = path.qbytes[i] / (q["median"] * 1e-6) / 1e9
        rows.append({"workload": work, "call": label, "gemm_us": g,
                     "gemm_tflops": round(fl / (g["median"] * 1e-6) / 1e12, 1),
                     "gemm_frac_fp8_peak": round(fl / (g["median"] * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
                     "gemm_min_hbm_gbs": round(by / (g["median"] * 1e-6) / 1e9, 1),
                     "quant_us": q, "quant_bytes": path.qbytes[i], "quant_gbs": round(qgbs, 1),
                     "quant_frac_hbm": round(qgbs / HBM_PEAK_GBS, 4)})
    return rows


def variant_breakdown(path, timer, reps):
    """GEMM and quantizer time of each variant next to the per-channel E4M3 call of the same
    shape (cache flushed before every repetition)."""
    from fp8_quantized_generative_amd import _lib
    rows = []
    for work, label, variant, fl, ref, fn in path.variants:
        g = stats_us(timer.kernel(fn, _lib.RQ_KERNEL_GEMM, reps))
        r = stats_us(timer.kernel(path.calls[ref][5], _lib.RQ_KERNEL_GEMM, reps))
        q = stats_us(timer.kernel(fn, _lib.RQ_KERNEL_QUANT, reps))
        rows.append({"workload": work, "call": label, "variant": variant, "gemm_us": g,
                     "gemm_tflops": round(fl / (g["median"] * 1e-6) / 1e12, 1),
                     "gemm_frac_fp8_peak": round(fl / (g["median"] * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
                     "quant_us": q, "reference_gemm_us": r})
    return rows


def cpu_baseline(target_s=12.0):
    """The CPU oracle on a bounded sample of the same workloads (rows sampled per linear)."""
    import workloads
    from oracle import ffn, linear, moe, quant
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    # offline weight quantization (untimed); the weights do not depend on the row count.
    # Four full-size experts serve the MoE sample.
    w2, w3, w4 = workloads.make(2, m=64), workloads.make(3, m=64), workloads.make(4, t=64, e=4)
    wqkv = quant.quantize_rows(w2["w_qkv"])
    wo = quant.quantize_rows(w2["w_o"])
    wgu = quant.quantize_rows(w3["w_gu"])
    wdn = quant.quantize_rows(w3["w_dn"])
    egu = [quant.quantize_rows(w4["w_gu"][e]) for e in range(4)]
    edn = [quant.quantize_rows(w4["w_dn"][e]) for e in range(4)]
    egu_q = np.stack([q for q, _ in egu]); egu_s = np.stack([s for _, s in egu])
    edn_q = np.stack([q for q, _ in edn]); edn_s = np.stack([s for _, s in edn])
    del w2, w3, w4

    def sample(rows):
        d2 = workloads.make(2, m=rows)
        d3 = workloads.make(3, m=rows)
        d4 = workloads.make(4, t=rows, e=4)
        flops = 0
        t0 = time.perf_counter()
        xq, xs = quant.quantize_rows(d2["x"])
        linear.linear(xq, xs, *wqkv)
        flops += 2 * rows * 6144 * 2048
        aq, as_ = quant.quantize_rows(d2["attn_out"])
        linear.linear(aq, as_, *wo)
        flops += 2 * rows * 2048 * 2048
        xq, xs = quant.quantize_rows(d3["x"])
        gu = linear.linear(xq, xs, *wgu)
        hq, hs = quant.quantize_rows(ffn.silu_mul(gu, 8192))
        linear.linear(hq, hs, *wdn)
        flops += 2 * rows * 16384 * 2048 + 2 * rows * 2048 * 8192
        r1 = moe.grouped_linear(d4["x"], moe.IN_TOKENS, moe.ACT_NONE, d4["ids"], egu_q, egu_s)
        moe.grouped_linear(r1["y"], moe.IN_PERMUTED, moe.ACT_SILU_MUL, d4["ids"], edn_q, edn_s,
                           moe.OUT_COMBINED, d4["topk_w"])
        flops += 2 * rows * 2 * 8192 * 2048 + 2 * rows * 2 * 2048 * 4096
        return flops, time.perf_counter() - t0

    # The oracle's cost is a fixed part (decoding each weight matrix) plus a part per row:
    # two short passes fit both, and the sample gets the rows that make it about target_s
    # seconds on this host.
    _, t_a = sample(64)
    _, t_b = sample(256)
    per_row = max((t_b - t_a) / 192, 1e-6)
    fixed = max(t_a - 64 * per_row, 0.0)
    rows = int(max(64, min(8192, (target_s - fixed) / per_row)) // 64 * 64)
    flops, dt = sample(rows)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle", "seconds": round(dt, 2),
            "sample": "%d token rows through each linear of the step: attention QKV and O, dense FFN "
                      "gate/up + SiLU + down, and the MoE expert FFN (F = 4096) over %d tokens, top-2 of 4 "
                      "full-size experts; float64 exact GEMMs; weights quantized beforehand (untimed); "
                      "rows sized from 64- and 256-row passes to about %.0f s" % (rows, rows, target_s)}


def cpu_router(tokens=16384):
    """The oracle router on the router workload (16384 tokens), in GB/s of its algorithmic bytes."""
    from oracle import router
    rng = np.random.default_rng(1104)
    x = (rng.standard_normal((tokens, 2048))).astype(np.float16)
    w = (rng.standard_normal((32, 2048)) / np.sqrt(2048)).astype(np.float16)
    t0 = time.perf_counter()
    router.route(x, w, 2)
    dt = time.perf_counter() - t0
    by = tokens * 2048 * 2 + 32 * 2048 * 2 + tokens * 2 * 6
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 3), "sample": "%d tokens x 2048, 32 experts, top-2" % tokens}


def cpu_attention(requests=128):
    """The oracle attention core on the attention workload (128 requests), in GB/s."""
    from oracle import attention
    rng = np.random.default_rng(2002)
    x = rng.standard_normal((requests * 32, 3 * 2048)).astype(np.float16)
    t0 = time.perf_counter()
    attention.attention(x, requests, 32, 16)
    dt = time.perf_counter() - t0
    by = x.size * 2 + requests * 32 * 2048 * 2
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "%d requests x 32 positions, 16 heads of 128" % requests}


def cpu_beam_topk():
    """The oracle top-k on the larger beam workload (32 x 262144, keep 512), in GB/s."""
    import workloads
    from oracle import topk
    s = workloads.beam_scores(np.random.default_rng(3512), 32, 512, 512)
    t0 = time.perf_counter()
    topk.topk(s, 512)
    dt = time.perf_counter() - t0
    by = s.size * 2 + 32 * 512 * 6
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 3), "sample": "32 requests x 512 beams x 512 codes, keep 512"}


def _find(path, patterns):
    import glob
    if not os.path.isdir(path):
        return path
    for pat in patterns:
        found = sorted(glob.glob(os.path.join(path, "**", pat), recursive=True))
        if found:
            return found[0]
    raise SystemExit("no rocprofv3 output (%s) under %s" % (", ".join(patterns), path))


def _rocprof_rows(path):
    """(kernel name, grid threads, workgroup threads, duration ns) of every dispatch, in launch order."""
    path = _find(path, ["*_results.db", "*kernel_trace.csv"])
    if path.endswith(".db"):
        import sqlite3
        db = sqlite3.connect(path)
        q = ("select name, grid_x * grid_y * grid_z, workgroup_x * workgroup_y * workgroup_z, duration "
             "from kernels order by start")
        return path, [(r[0], int(r[1]), int(r[2]), int(r[3])) for r in db.execute(q)]
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1)) * int(r.get("Grid_Size_Z", 1))
            wg = int(r["Workgroup_Size_X"]) * int(r.get("Workgroup_Size_Y", 1)) * int(r.get("Workgroup_Size_Z", 1))
            rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"], grid, wg,
                         int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    return path, [r[1:] for r in rows]


_KIND_TOKEN = {"quant": "quant_rows", "gemm": "gemm_fp8_kernel", "reduce": "splitk_reduce", "plan": "plan_single",
               "plan_hist": "plan_hist", "plan_scan": "plan_scan", "plan_scatter": "plan_scatter",
               "combine": "combine_kernel"}


def _align_steps(names, only, steps):
    """Indices (into names) of the dispatches of the last `steps` steps, with their labels.

    names: kernel names in launch order.  Only this library's kernels are considered; the
    step's kernel sequence is matched backwards from the last one (after the timed steps the
    profiled command launches none of them)."""
    seq = step_dispatches(only)
    ours = [i for i, n in enumerate(names) if any(k in n for k in OUR_KERNELS)]
    period = len(seq)
    if steps is None:
        steps = 0
        while (steps + 1) * period <= len(ours):
            block = ours[len(ours) - (steps + 1) * period:len(ours) - steps * period]
            if not all(_KIND_TOKEN[seq[j][1]] in names[block[j]] for j in range(period)):
                break
            steps += 1
    if steps <= 0 or steps * period > len(ours):
        raise SystemExit("could not find the step's kernel sequence in the profile")
    picked = ours[len(ours) - steps * period:]
    out = []
    for j, idx in enumerate(picked):
        label, kind = seq[j % period]
        if _KIND_TOKEN[kind] not in names[idx]:
            raise SystemExit("dispatch %d (%s) does not match %s %s" % (idx, names[idx], label, kind))
        out.append((idx, label, kind))
    return out, steps


def rocprof_summary(path, only=None, steps=None):
    src, rows = _rocprof_rows(path)
    names = [r[0] for r in rows]
    aligned, nsteps = _align_steps(names, only, steps)
    groups = {}
    for idx, label, kind in aligned:
        groups.setdefault((label, kind), []).append(rows[idx][3])
    step_ns = sum(sum(v) for v in groups.values()) / nsteps
    print("# rocprofv3 kernel trace: %s (%d steps matched)" % (os.path.basename(src), nsteps))
    print("# sum of kernel durations per step: %.1f us" % (step_ns / 1e3))
    print("# %-28s %-13s %6s %10s %10s %10s %6s" % ("call", "kernel", "calls", "avg_us", "min_us", "max_us", "pct"))
    for (label, kind), durs in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print("  %-28s %-13s %6d %10.2f %10.2f %10.2f %5.1f%%" % (
            label, kind, len(durs), np.mean(durs) / 1e3, min(durs) / 1e3, max(durs) / 1e3,
            100.0 * sum(durs) / (step_ns * nsteps)))
    dom = groups.get(("%s %s" % DOMINANT, "gemm"))
    if dom:
        print("# dominant launch (%s %s grouped GEMM) sources sha256_16: %s" % (DOMINANT[0], DOMINANT[1],
                                                                           source_hash(GEMM_SOURCES)))
        print("# dominant launch (%s %s grouped GEMM): avg %.2f us over %d calls" % (
            DOMINANT[0], DOMINANT[1], np.mean(dom) / 1e3, len(dom)))


def _pmc_rows(path, counter):
    """(kernel name, counter value summed over the dispatch's instances) per dispatch, in order."""
    import csv
    path = _find(path, ["*counter_collection.csv"])
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = per.get(d, (r["Kernel_Name"], 0.0))
            per[d] = (name, v + float(r["Counter_Value"]))
    return [per[d] for d in sorted(per)]


def _pmc_db(path):
    """{dispatch_id: (kernel name, duration ns, {counter: value summed over instances})} from a
    rocprofv3 --pmc database."""
    import sqlite3
    path = _find(path, ["*_results.db"])
    db = sqlite3.connect(path)
    per = {}
    q = ("select dispatch_id, kernel_name, max(duration), counter_name, sum(value) from counters_collection "
         "group by dispatch_id, counter_name")
    for d, name, dur, cn, v in db.execute(q):
        e = per.setdefault(int(d), [name, int(dur), {}])
        e[2][cn] = float(v)
    return path, per


XCDS, SIMDS = 8, 1024  # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs


def pmc_summary(path, only=None, steps=None):
    """Per call of the step: FP8 MFMA instructions and flops executed (against the algorithmic
    flops), the MFMA pipe's busy fraction and the engine clock, from a --pmc run with
    SQ_INSTS_VALU_MFMA_MOPS_F8, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE."""
    import workloads
    src, per = _pmc_db(path)
    ids = sorted(per)
    names = [per[d][0] for d in ids]
    aligned, nsteps = _align_steps(names, only, steps)
    flops = {}
    for wl, label, shapes in (("attention", ("qkv", "o"), workloads.gemm_shapes(2)),
                              ("ffn", ("gate_up", "down"), workloads.gemm_shapes(3)),
                              ("moe", ("gate_up", "down"), workloads.gemm_shapes(4)),
                              ("layer_small_m", ("qkv", "o", "gate_up", "down", "moe_gate_up", "moe_down"),
                               workloads.gemm_shapes(5))):
        for lb, (m, n, k) in zip(label, shapes):
            flops["%s %s" % (wl, lb)] = 2 * m * n * k
    groups = {}
    for idx, label, kind in aligned:
        if kind == "gemm":
            groups.setdefault(label, []).append(per[ids[idx]])
    print("# rocprofv3 --pmc: %s (%d steps matched)" % (os.path.basename(src), nsteps))
    print("# %-26s %8s %9s %10s %8s %7s %9s %7s %8s" % (
        "call", "avg_us", "clock_GHz", "mfma_f8", "exec/alg", "busy", "TFLOP/s", "frac5P", "valu/mfma"))
    for label, recs in groups.items():
        dur = np.mean([r[1] for r in recs])
        c = {k: np.mean([r[2].get(k, np.nan) for r in recs]) for k in recs[0][2]}
        ghz = c.get("GRBM_GUI_ACTIVE", np.nan) / XCDS / dur
        executed = c.get("SQ_INSTS_VALU_MFMA_MOPS_F8", np.nan) * 512
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", np.nan) / (SIMDS * c.get("GRBM_GUI_ACTIVE", np.nan) / XCDS)
        alg = flops.get(label, np.nan)
        valu = (c.get("SQ_INSTS_VALU", np.nan) - c.get("SQ_INSTS_VALU_MFMA_F8", 0)) / c.get("SQ_INSTS_VALU_MFMA_F8", np.nan)
        print("  %-26s %8.1f %9.3f %10.0f %8.3f %7.3f %9.1f %7.3f %8.2f" % (
            label, dur / 1e3, ghz, c.get("SQ_INSTS_VALU_MFMA_F8", np.nan), executed / alg, busy,
            alg / dur / 1e3, alg / dur / 1e3 / FP8_PEAK_TFLOPS, valu))
    print("# clock = GRBM_GUI_ACTIVE / %d XCDs / duration; exec/alg = MOPS_F8 * 512 / (2 M N K over real rows); "
          "busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs * GRBM_GUI_ACTIVE / %d); valu/mfma = non-MFMA VALU "
          "instructions per FP8 MFMA" % (XCDS, SIMDS, XCDS))


CUS = 256  # MI355X compute units: TA, TD and TCP counters are summed over them


def pmc_dump(paths, only=None, steps=None):
    """Every counter of one or more rocprofv3 --pmc databases, averaged per GEMM call of the
    step (the same dispatch matching as --pmc-summary), with the GEMM's average duration, then
    the derived memory-pipeline figures of each call."""
    derived = {}
    for path in paths:
        src, per = _pmc_db(path)
        ids = sorted(per)
        aligned, nsteps = _align_steps([per[d][0] for d in ids], only, steps)
        groups = {}
        for idx, label, kind in aligned:
            if kind == "gemm":
                groups.setdefault(label, []).append(per[ids[idx]])
        print("# rocprofv3 --pmc: %s (%d steps matched)" % (path, nsteps))
        for label, recs in groups.items():
            print("  %-26s avg_us %.1f" % (label, np.mean([r[1] for r in recs]) / 1e3))
            c = {k: float(np.mean([r[2][k] for r in recs])) for k in sorted(recs[0][2])}
            for k, v in c.items():
                print("    %-34s %16.0f" % (k, v))
            d = derived.setdefault(label, {})
            cyc = c.get("GRBM_GUI_ACTIVE", np.nan) / XCDS  # engine cycles of the dispatch
            for name, key in (("ta_busy", "TA_TA_BUSY"), ("td_busy", "TD_TD_BUSY"), ("td_tc_stall", "TD_TC_STALL"),
                              ("tcp_pending_stall", "TCP_PENDING_STALL_CYCLES")):
                if key in c:
                    d[name] = c[key] / (CUS * cyc)
            if "TCP_TCC_READ_REQ" in c and "TCP_TCC_READ_REQ_LATENCY" in c:
                d["l2_read_latency_cycles"] = c["TCP_TCC_READ_REQ_LATENCY"] / c["TCP_TCC_READ_REQ"]
                d["l2_read_req_per_cu_cycle"] = c["TCP_TCC_READ_REQ"] / (CUS * cyc)
            if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
                d["l2_hit_rate"] = c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
            for name, key in (("lds_idx_active", "SQ_LDS_IDX_ACTIVE"), ("lds_bank_conflict", "SQ_LDS_BANK_CONFLICT"),
                              ("lds_wait_inst", "SQ_WAIT_INST_LDS")):
                if key in c:
                    d[name] = c[key] / (CUS * cyc)
    cols = ("ta_busy", "td_busy", "td_tc_stall", "tcp_pending_stall", "l2_read_latency_cycles",
            "l2_read_req_per_cu_cycle", "l2_hit_rate", "lds_idx_active", "lds_bank_conflict", "lds_wait_inst")
    print("# derived per GEMM call: busy/stall fractions = counter / (%d CUs x GRBM_GUI_ACTIVE / %d XCDs) (the LDS "
          "ones too); L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (cycles); L2 hit rate = TCC_HIT / "
          "(TCC_HIT + TCC_MISS)" % (CUS, XCDS))
    print("# %-26s %s" % ("call", " ".join("%12s" % c[:12] for c in cols)))
    for label, d in derived.items():
        print("  %-26s %s" % (label, " ".join("%12.3f" % d.get(c, np.nan) for c in cols)))


def source_hash(files):
    """Hash of a kernel's code: stored traffic counters and traces are valid only for this code.
    Line comments and blank lines are left out (the sources use no block comments and no "//"
    inside string literals), so editing a comment keeps the stored evidence valid."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp8_quantized_generative_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()[:16]


GEMM_SOURCES = ("gemm.hip", "common.h")
QUANT_SOURCES = ("quant.hip", "common.h")
QUANT_CALL = ("moe", "down")   # the largest row-quantizer call: 32768 permuted rows x 4096


def gemm_source_hash():
    return source_hash(GEMM_SOURCES)


def dominant_algorithmic_bytes():
    """Bytes the MoE gate/up grouped GEMM must move at least once: its FP8 A rows (one per
    routed slot) and expert weights, the FP32 scales, and its FP16 output h = silu(g) * u
    (F columns per routed slot; the gated layout never writes g and u)."""
    t, k, f, e, top_k = 16384, 2048, 4096, 32, 2
    r, n = t * top_k, 2 * f
    return r * k + e * n * k + 4 * (r + e * n) + 2 * r * f


def quant_algorithmic_bytes():
    """The row quantizer of the MoE down call: FP16 rows in, E4M3 rows and FP32 scales out."""
    r, k = 16384 * 2, 4096
    return 2 * r * k + r * k + 4 * r


def traffic_summary(fetch_dir, write_dir, out, only=None, steps=None):
    """Per-launch counter values of the dominant GEMM and of the largest quantizer call, and
    of the calibration copy that follows the profiled steps."""
    gemm = {"kernel": "gemm_fp8_kernel (grouped, 256x256) for the %s %s call" % DOMINANT,
            "source_sha256_16": source_hash(GEMM_SOURCES)}
    qnt = {"kernel": "quant_rows for the %s %s call (32768 x 4096 FP16 rows)" % QUANT_CALL,
           "source_sha256_16": source_hash(QUANT_SOURCES)}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        names = [r[0] for r in rows]
        aligned, nsteps = _align_steps(names, only, steps)
        last = max(i for i, _, _ in aligned)
        # the calibration copy (x * 1, an elementwise multiply); the fills that allocate the
        # flush and calibration buffers around it are not copies
        copies = [r for r in rows[last + 1:] if "MulFunctor" in r[0]]
        for res, label, kind in ((gemm, "%s %s" % DOMINANT, "gemm"), (qnt, "%s %s" % QUANT_CALL, "quant")):
            vals = [rows[i][1] for i, lb, kd in aligned if lb == label and kd == kind]
            if not vals or not copies:
                raise SystemExit("%s: %s %s launch or calibration copy not found" % (counter, label, kind))
            res[counter.lower() + "_kib_per_launch"] = round(float(np.mean(vals)), 1)
            res[counter.lower() + "_launches"] = len(vals)
            res["copy_" + counter.lower() + "_kib"] = round(copies[-1][1], 1)
            res["copy_kernel"] = copies[-1][0][:120]
    return gemm, qnt


def finish_traffic(result, copy_mib, out, algorithmic):
    copy_bytes = copy_mib * 1024 * 1024
    result["copy_mib"] = copy_mib
    f_fac = result["copy_fetch_size_kib"] * 1024 / copy_bytes
    w_fac = result["copy_write_size_kib"] * 1024 / copy_bytes
    result["fetch_factor"] = round(f_fac, 4)
    result["write_factor"] = round(w_fac, 4)
    traffic = (result["fetch_size_kib_per_launch"] * 1024 / f_fac +
               result["write_size_kib_per_launch"] * 1024 / w_fac)
    result["traffic_bytes_per_launch"] = int(traffic)
    result["algorithmic_bytes_per_launch"] = algorithmic
    result["traffic_over_algorithmic"] = round(traffic / algorithmic, 3)
    with open(out, "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result, indent=1))


GEMM_TRAFFIC = os.path.join(ROOT, "profiles", "gemm_fp8_grouped_moe_gate_up_traffic.json")
QUANT_TRAFFIC = os.path.join(ROOT, "profiles", "quant_rows_moe_down_traffic.json")


def stored_traffic(path=GEMM_TRAFFIC, sources=GEMM_SOURCES):
    """HBM bytes per launch from a committed counter summary, or None when it is missing or
    was taken on different kernel sources."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(sources):
        return None
    return t.get("traffic_bytes_per_launch")


STEP_TRACE = os.path.join(ROOT, "profiles", "bench_step_kernels.txt")


def stored_trace_us(path=STEP_TRACE, sources=GEMM_SOURCES):
    """The dominant launch's average duration in the committed kernel trace of the step, or None
    when it is missing or was taken on different GEMM sources."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = [l.rsplit(":", 1)[1].strip() for l in lines if l.startswith("# dominant launch") and "sha256_16" in l]
    avg = [l for l in lines if l.startswith("# dominant launch") and " avg " in l]
    if not sha or not avg or sha[0] != source_hash(sources):
        return None
    try:
        return float(avg[0].split(" avg ")[1].split(" us")[0])
    except (IndexError, ValueError):
        return None


def kernel_stats(path):
    """Per-instantiation statistics of this library's kernels from rocprofv3 --stats."""
    import csv
    src = _find(path, ["*kernel_stats.csv"])
    rows = []
    with open(src) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if not any(k in name for k in OUR_KERNELS + ("router_topk", "attention_core", "topk_segment", "pack_slabs",
                                                       "quant_blocks", "tensor_")):
                continue
            short = name.replace("rq::(anonymous namespace)::", "").replace("void ", "")
            short = short.split("(")[0] if "(" in short else short
            rows.append((float(r["TotalDurationNs"]), int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), short))
    rows.sort(reverse=True)
    print("# rocprofv3 kernel statistics: %s" % os.path.basename(src))
    print("# %6s %10s %10s %10s  %s" % ("calls", "avg_us", "min_us", "max_us", "kernel"))
    for total, calls, avg, mn, mx, name in rows:
        print("  %6d %10.2f %10.2f %10.2f  %s" % (calls, avg / 1e3, mn / 1e3, mx / 1e3, name))


def main():
    args = parse()
    if args.kernel_stats:
        kernel_stats(args.kernel_stats)
        return
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.only, args.steps_in_profile)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.only, args.steps_in_profile)
        return
    if args.pmc_dump:
        pmc_dump(args.pmc_dump, args.only, args.steps_in_profile)
        return
    if args.traffic_summary:
        fetch_dir, write_dir, out = args.traffic_summary
        gemm, qnt = traffic_summary(fetch_dir, write_dir, out, args.only, args.steps_in_profile)
        finish_traffic(gemm, args.calibrate_copy_mb or 512, out, dominant_algorithmic_bytes())
        finish_traffic(qnt, args.calibrate_copy_mb or 512, os.path.join(os.path.dirname(out) or ".",
                                                                        os.path.basename(QUANT_TRAFFIC)),
                       quant_algorithmic_bytes())
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_quantized_generative_amd as rq
    from fp8_quantized_generative_amd import _lib

    torch.cuda.set_device(0)
    hip = Hip()
    print("[bench] building inputs", file=sys.stderr, flush=True)
    path = Path(rq, torch, args.only, variants=not args.no_variants, wlayout=args.wlayout)
    print("[bench] %d calls per step, %.1f GFLOP" % (len(path.calls), path.flops / 1e9), file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    qevs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        path.step(hooks=((path.dominant, _lib.RQ_KERNEL_GEMM, evs[s][0], evs[s][1]),
                         (path.quant_dominant, _lib.RQ_KERNEL_QUANT, qevs[s][0], qevs[s][1])))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = path.flops * args.steps / elapsed / 1e12
    print("[bench] timed %d steps: %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)

    # the dominant kernel inside the timed steps (cache state as the step leaves it)
    dom = path.calls[path.dominant]
    dom_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    dom_st = stats_us(dom_ms)
    achieved = dom[3] / (dom_st["mean"] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": stored_traffic(),
                "algorithmic_bytes": dominant_algorithmic_bytes(),
                "kernel": "gemm_fp8_kernel<grouped> (%s %s)" % (dom[0], dom[1]),
                "flops_per_launch": dom[3], "avg_launch_us": dom_st["mean"],
                "launch_us_in_step": dom_st,
                "frac_at_median": round(dom[3] / (dom_st["median"] * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
                "trace_avg_us": stored_trace_us(),
                "timing": "HIP events around each launch inside the %d timed steps (cache-warm: the "
                          "step's previous kernels leave the quantized A rows in cache); achieved = "
                          "flops / mean launch time; trace_avg_us / frac_trace: the same kernel's average in "
                          "the committed rocprofv3 trace of the step (profiles/bench_step_kernels.txt), "
                          "given while it was taken on these GEMM sources" % args.steps}
    if roofline["trace_avg_us"]:
        roofline["frac_trace"] = round(dom[3] / (roofline["trace_avg_us"] * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)

    qcall = path.calls[path.quant_dominant]
    q_st = stats_us([hip.elapsed_ms(a, b) for a, b in qevs])
    q_gbs = path.qbytes[path.quant_dominant] / (q_st["mean"] * 1e-6) / 1e9
    quant_roofline = {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                      "traffic": (stored_traffic(QUANT_TRAFFIC, QUANT_SOURCES)
                                  if (qcall[0], qcall[1]) == QUANT_CALL else None),
                      "kernel": "quant_rows (%s %s)" % (qcall[0], qcall[1]),
                      "bytes_per_launch": path.qbytes[path.quant_dominant], "avg_launch_us": q_st["mean"],
                      "launch_us_in_step": q_st,
                      "timing": "in-step HIP events, cache-warm (its input was just written by the previous "
                                "GEMM); the flushed figures are under quant_targets"}

    result = {
        "metric": "FP8 linear TFLOP/s (dense + MoE grouped) and % of MI355X FP8 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, fp16 out)",
        "data": "synthetic",
        "frac_fp8_peak": round(value / FP8_PEAK_TFLOPS, 4),
        "config": {"workload": "+".join(path.config) + " (full-size W8A8 FP8 linears, one step each)",
                   **path.config, "gflop_per_step": round(path.flops / 1e9, 2),
                   "weight_layout": ("slabs [K/64][N][64] (rq_fp8_pack_weights, offline)"
                                     if path.wlayout == "slabs" else "rows [N][K]")},
        "roofline": roofline,
        "quant_roofline": quant_roofline,
    }
    if args.calibrate_copy_mb:
        # an elementwise kernel that reads and writes exactly n bytes (a plain copy, x * 1); a
        # 1 GiB write in between evicts the source from the 256 MB last-level cache first
        n = args.calibrate_copy_mb * 1024 * 1024
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(2.0)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst, flush
    flush = Flush(torch)
    timer = KernelTimer(hip, torch, flush)
    reps = max(args.reps, 1)
    if not args.no_kernels:
        print("[bench] per-kernel breakdown (flushed, %d reps each)" % reps, file=sys.stderr, flush=True)
        result["kernels"] = kernel_breakdown(path, timer, reps)
        by_call = {(r["workload"], r["call"]): r for r in result["kernels"]}
        # the three row-quantizer instances held to the >= 70% HBM target, flushed
        targets = []
        for key, what in ((("ffn", "down"), "FFN h re-quantization, 4096 x 8192 (SiLU*up written by the gate/up GEMM)"),
                          (("moe", "gate_up"), "MoE token quantization, 16384 x 2048, one row per routed slot"),
                          (("moe", "down"), "MoE h re-quantization, 32768 x 4096 permuted rows")):
            r = by_call.get(key)
            if r is not None:
                targets.append({"call": "%s %s" % key, "what": what, "bytes": r["quant_bytes"],
                                "us": r["quant_us"], "gbs": r["quant_gbs"], "frac_hbm": r["quant_frac_hbm"]})
        if targets:
            result["quant_targets"] = {"timing": "isolated, L2 and last-level cache flushed (a 1 GiB read) "
                                                 "before each of %d repetitions; GB/s from the median" % reps,
                                       "instances": targets}
    # the small dense linear (quantizer + GEMM) and the small-M layer as a whole, flushed
    layer = [c for c in path.calls if c[0] == "layer_small_m"]
    if not args.no_kernels:
        fl1, fn1 = path.c1
        g1 = stats_us(timer.kernel(fn1, _lib.RQ_KERNEL_GEMM, reps))
        q1 = stats_us(timer.kernel(fn1, _lib.RQ_KERNEL_QUANT, reps))
        result["dense_small"] = {"workload": "64 x 512 x 512 dense linear (quantizer + GEMM)",
                                 "kernels_us": round(g1["median"] + q1["median"], 2), "gemm_us": g1, "quant_us": q1,
                                 "call_us_with_host_dispatch": stats_us(timer.sequence([fn1], reps)),
                                 "timing": "HIP events around each kernel, flushed before each repetition; the whole "
                                           "call timed from Python includes the binding's host dispatch"}
    if layer and not args.no_kernels:
        lay = stats_us(timer.sequence([c[5] for c in layer], reps))
        lay_bytes = sum(c[4] for c in layer)
        result["layer_small_m"] = {
            "workload": path.config["layer_small_m"], "us": lay, "min_hbm_bytes": lay_bytes,
            "hbm_floor_us": round(lay_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
            "gbs": round(lay_bytes / (lay["median"] * 1e-6) / 1e9, 1),
            "frac_hbm": round(lay_bytes / (lay["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "the six calls back to back, flushed before each repetition; bytes = weights of the "
                      "touched experts + each call's FP16 input and output"}
    if path.variants:
        print("[bench] variants", file=sys.stderr, flush=True)
        result["variants"] = variant_breakdown(path, timer, min(reps, 20))
    for key, kind, what in (("router", _lib.RQ_KERNEL_ROUTER, "MoE router: 16384 tokens x 2048 FP16, 32 experts, top-2"),
                            ("attention_core", _lib.RQ_KERNEL_ATTENTION,
                             "attention core: 128 requests x 32 positions, 16 heads of 128, causal, FP16")):
        item = path.router if key == "router" else path.attention
        if item is None:
            continue
        by, fn = item
        st = stats_us(timer.kernel(fn, kind, reps))
        result[key] = {"workload": what, "us": st, "bytes_per_launch": by,
                       "achieved_gbs": round(by / (st["median"] * 1e-6) / 1e9, 1),
                       "frac_hbm": round(by / (st["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "timing": "flushed before each repetition"}
    if path.beam:
        rows = []
        for what, by, fn, default in path.beam:
            st = stats_us(timer.kernel(fn, _lib.RQ_KERNEL_TOPK, reps))
            rows.append({"workload": what, "us": st, "bytes_per_call": by,
                         "achieved_gbs": round(by / (st["median"] * 1e-6) / 1e9, 1),
                         "frac_hbm": round(by / (st["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "torch_topk_us": stats_us(timer.sequence([default], reps))["median"]})
        result["beam_topk"] = {"timing": "HIP events around all kernels of the call (every stage), flushed before "
                                         "each repetition; bytes = FP16 scores read + int32 index and FP16 score of "
                                         "each pick written",
                               "workloads": rows}
    del flush, timer
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        del path
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline()
        for key, fn in (("router", cpu_router), ("attention_core", cpu_attention), ("beam_topk", cpu_beam_topk)):
            if key in result:
                result[key]["cpu_oracle"] = fn()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
