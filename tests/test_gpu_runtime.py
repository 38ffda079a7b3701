"""Runtime behaviour of the C ABI on the GPU: the device error word for routing ids outside
[0, E), and calls on a stream other than the current one.

The error-word case passes out-of-range ids on purpose: the host cannot see device ids, so
the routing-plan kernel reports them (RQ_FLAG_EXPERT_ID) and maps them into [0, E) so that
every kernel of the call stays in bounds and exits normally.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import case, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def test_expert_id_out_of_range_sets_flag():
    rq = require_gpu()
    case("moe: routing ids outside [0, E) set the device error word")
    d = workloads.make(4, t=96, k=128, f=64, e=6)
    w_q, w_s = rq.quant_weights(dev(d["w_gu"]))
    x = dev(d["x"])
    rq.debug_flag(clear=True)
    good = dev(d["ids"].astype(np.int32))
    y_good = host(rq.moe_grouped_linear(x, good, w_q, w_s))
    assert rq.debug_flag() == 0
    for bad_id in (6, -1, 1 << 30):
        ids = d["ids"].astype(np.int32).copy()
        ids[17, 1] = bad_id
        y = rq.moe_grouped_linear(x, dev(ids), w_q, w_s)
        torch.cuda.synchronize()
        assert y.shape == y_good.shape
        flags = rq.debug_flag(clear=True)
        assert flags & rq.RQ_FLAG_EXPERT_ID, (bad_id, flags)
        assert rq.debug_flag() == 0
    # the word stays clear for valid routing, and results are unchanged
    y2 = host(rq.moe_grouped_linear(x, good, w_q, w_s))
    assert rq.debug_flag() == 0
    assert np.array_equal(y_good.view(np.uint16), y2.view(np.uint16))


def test_calls_on_a_side_stream():
    """Every entry point run on a stream that is not the current one gives the bytes it gives
    on the current stream; buffers the binding allocates belong to that stream."""
    rq = require_gpu()
    case("linear and moe on a side stream")
    d = workloads.make(4, t=300, k=256, f=128, e=8)
    w_q, w_s = rq.quant_weights(dev(d["w_gu"]))
    x, ids, tw = dev(d["x"]), dev(d["ids"].astype(np.int32)), dev(d["topk_w"])
    wl_q, wl_s = rq.quant_weights(dev(d["w_gu"][3]))
    ref_lin = host(rq.linear(x, wl_q, wl_s))
    ref_moe = host(rq.moe_grouped_linear(x, ids, w_q, w_s))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(rq.linear(x, wl_q, wl_s, stream=side))
        outs.append(rq.moe_grouped_linear(x, ids, w_q, w_s, stream=side))
        # freed at once on the host: the allocator may only reuse them for later side-stream work
        rq.linear(x, wl_q, wl_s, stream=side)
    q2, s2 = rq.quant_weights(dev(d["w_gu"][3]), stream=side)
    side.synchronize()
    for i, o in enumerate(outs):
        ref = ref_lin if i % 2 == 0 else ref_moe
        assert np.array_equal(host(o).view(np.uint16), ref.view(np.uint16))
    assert torch.equal(q2, wl_q) and torch.equal(s2, wl_s)


def test_concurrent_host_threads():
    """Calls from several host threads at once, each on its own stream with its own buffers
    and workspaces (the header's thread-safety contract): every result equals the
    single-threaded one, bit for bit."""
    import threading

    rq = require_gpu()
    case("linear and moe from 4 host threads on 4 streams")
    d = workloads.make(4, t=400, k=256, f=128, e=8)
    w_q, w_s = rq.quant_weights(dev(d["w_gu"]))
    w_p = rq.pack_weights(w_q)
    x, ids = dev(d["x"]), dev(d["ids"].astype(np.int32))
    wl_q, wl_s = rq.quant_weights(dev(d["w_gu"][5]))
    ref_lin = host(rq.linear(x, wl_q, wl_s))
    ref_moe = host(rq.moe_grouped_linear(x, ids, w_p, w_s, wlayout="slabs"))
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = [[] for _ in streams]
    errors = []

    def work(n):
        try:
            s = streams[n]
            with torch.cuda.stream(s):
                for _ in range(6):
                    results[n].append(("lin", rq.linear(x, wl_q, wl_s, stream=s)))
                    results[n].append(("moe", rq.moe_grouped_linear(x, ids, w_p, w_s, wlayout="slabs", stream=s)))
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(n,)) for n in range(len(streams))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for s in streams:
        s.synchronize()
    for rs in results:
        assert len(rs) == 12
        for kind, o in rs:
            ref = ref_lin if kind == "lin" else ref_moe
            assert np.array_equal(host(o).view(np.uint16), ref.view(np.uint16))
