"""The C ABI library loads, exports every symbol the header declares, and rejects bad
arguments on the host with the documented status codes before touching a device.

No compute call is made here (no GPU): every case fails validation, or is a documented
no-op (zero rows), which returns before any device query.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq_fp8.h")

lib_mod = pytest.importorskip("fp8_quantized_generative_amd._lib")

if not os.path.exists(lib_mod.LIB_PATH):
    pytest.skip("librq_fp8.so not built", allow_module_level=True)

RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_ALIGN, RQ_ERR_WORKSPACE, RQ_ERR_ARG = 1, 2, 3, 4, 7
FAKE = 0x10000  # a 16-byte-aligned, never dereferenced "device" address


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = ctypes.CDLL(lib_mod.LIB_PATH)
    names = _declared_symbols()
    assert "rq_fp8_linear" in names and "rq_fp8_moe_grouped_linear" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(lib_mod.SIGNATURES)


def test_status_strings():
    lib = lib_mod.load()
    assert lib.rq_status_string(0) == b"ok"
    assert lib.rq_status_string(4) == b"workspace too small"
    assert lib.rq_status_string(99) == b"unknown status"


def test_workspace_sizes():
    lib = lib_mod.load()
    assert lib.rq_fp8_linear_workspace_size(4096, 2048, 0) == 4096 * 2048 + 4096 * 4
    assert lib.rq_fp8_linear_workspace_size(3, 16, 0) == 256 + 256
    assert lib.rq_fp8_linear_workspace_size(-1, 16, 0) == 0
    # split-K partial sums only for few rows and long K: 512 x 2048 x 8192 splits K in 4,
    # 300 x 6144 x 4096 in 2; K = 2048 and 4096 rows do not split
    assert lib.rq_fp8_linear_workspace_size_ex(512, 2048, 8192, 2) == 512 * 8192 + 2048 + 4 * 512 * 2048 * 4
    assert lib.rq_fp8_linear_workspace_size_ex(300, 6144, 4096, 0) == \
        300 * 4096 + 1280 + 2 * 300 * 6144 * 4
    assert lib.rq_fp8_linear_workspace_size_ex(512, 2048, 2048, 0) == lib.rq_fp8_linear_workspace_size(512, 2048, 0)
    assert lib.rq_fp8_linear_workspace_size_ex(512, 16384, 2048, 0) == lib.rq_fp8_linear_workspace_size(512, 2048, 0)
    assert lib.rq_fp8_linear_workspace_size_ex(4096, 2048, 8192, 0) == lib.rq_fp8_linear_workspace_size(4096, 8192, 0)
    assert lib.rq_fp8_linear_workspace_size_ex(64, 512, 512, 0) == lib.rq_fp8_linear_workspace_size(64, 512, 0)
    assert lib.rq_fp8_linear_workspace_size_ex(512, 2048, 2048 + 16, 0) == lib.rq_fp8_linear_workspace_size(512, 2064, 0)
    assert lib.rq_fp8_linear_workspace_size_ex(512, 0, 2048, 0) == 0
    a = lib.rq_fp8_moe_workspace_size(16384, 2, 32, 8192, 2048, 0, 0, 0)
    b = lib.rq_fp8_moe_workspace_size(16384, 2, 32, 2048, 4096, 1, 1, 1)
    assert a >= 16384 * 2048 and b >= 32768 * 4096 + 32768 * 2048 * 2


def _linear(**kw):
    args = dict(x=FAKE, M=64, K=512, act=0, w_q=FAKE, w_scale=FAKE, N=512, y=FAKE,
                ws=FAKE, ws_bytes=1 << 30, dbg=None, stream=None)
    args.update(kw)
    lib = lib_mod.load()
    return lib.rq_fp8_linear(args["x"], args["M"], args["K"], args["act"], args["w_q"], args["w_scale"],
                             args["N"], args["y"], args["ws"], args["ws_bytes"], args["dbg"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(act=3), RQ_ERR_ARG),
    (dict(act=2, N=96), RQ_ERR_ALIGN),
    (dict(M=-1), RQ_ERR_SHAPE),
    (dict(K=0), RQ_ERR_SHAPE),
    (dict(N=-16), RQ_ERR_SHAPE),
    (dict(K=24), RQ_ERR_ALIGN),
    (dict(N=40), RQ_ERR_ALIGN),
    (dict(w_q=None), RQ_ERR_NULL),
    (dict(w_scale=None), RQ_ERR_NULL),
    (dict(x=None), RQ_ERR_NULL),
    (dict(y=None), RQ_ERR_NULL),
    (dict(x=FAKE + 8), RQ_ERR_ALIGN),
    (dict(y=FAKE + 2), RQ_ERR_ALIGN),
    (dict(w_scale=FAKE + 2), RQ_ERR_ALIGN),
    (dict(ws_bytes=64 * 512), RQ_ERR_WORKSPACE),
    (dict(ws=None), RQ_ERR_WORKSPACE),
])
def test_linear_rejects(kw, code):
    assert _linear(**kw) == code


def test_linear_zero_rows_is_noop():
    assert _linear(M=0, x=None, y=None, ws=None, ws_bytes=0) == 0


def test_linear_debug_buffers_replace_workspace():
    d = lib_mod.DebugOut(FAKE, FAKE + 4, 0)
    assert _linear(M=0, dbg=ctypes.byref(d)) == 0
    d = lib_mod.DebugOut(FAKE + 4, 0, 0)
    assert _linear(dbg=ctypes.byref(d)) == RQ_ERR_ALIGN


def _moe(**kw):
    args = dict(x=FAKE, il=0, act=0, ids=FAKE, w=FAKE, T=128, top_k=2, w_q=FAKE, w_scale=FAKE,
                E=8, N=64, K=64, y=FAKE, ol=0, ws=FAKE, ws_bytes=1 << 30, dbg=None, stream=None)
    args.update(kw)
    lib = lib_mod.load()
    return lib.rq_fp8_moe_grouped_linear(args["x"], args["il"], args["act"], args["ids"], args["w"], args["T"],
                                         args["top_k"], args["w_q"], args["w_scale"], args["E"], args["N"],
                                         args["K"], args["y"], args["ol"], args["ws"], args["ws_bytes"],
                                         args["dbg"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(il=2), RQ_ERR_ARG),
    (dict(ol=5), RQ_ERR_ARG),
    (dict(act=-1), RQ_ERR_ARG),
    (dict(act=3), RQ_ERR_ARG),
    (dict(act=2, N=96), RQ_ERR_ALIGN),
    (dict(T=-1), RQ_ERR_SHAPE),
    (dict(E=0), RQ_ERR_SHAPE),
    (dict(E=1025), RQ_ERR_SHAPE),
    (dict(top_k=0), RQ_ERR_SHAPE),
    (dict(top_k=9), RQ_ERR_SHAPE),
    (dict(K=40), RQ_ERR_ALIGN),
    (dict(N=8), RQ_ERR_ALIGN),
    (dict(ids=None), RQ_ERR_NULL),
    (dict(w_q=None), RQ_ERR_NULL),
    (dict(ol=1, w=None), RQ_ERR_ARG),
    (dict(ids=FAKE + 2), RQ_ERR_ALIGN),
    (dict(ws_bytes=100), RQ_ERR_WORKSPACE),
])
def test_moe_rejects(kw, code):
    assert _moe(**kw) == code


def test_moe_zero_tokens_is_noop():
    assert _moe(T=0, x=None, ids=None, y=None, ws=None, ws_bytes=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), RQ_ERR_SHAPE),
    (dict(K=8), RQ_ERR_ALIGN),
    (dict(w=None), RQ_ERR_NULL),
    (dict(w_scale=FAKE + 1), RQ_ERR_ALIGN),
])
def test_quant_weights_rejects(kw, code):
    args = dict(w=FAKE, B=1, N=64, K=64, w_q=FAKE, w_scale=FAKE, stream=None)
    args.update(kw)
    lib = lib_mod.load()
    assert lib.rq_fp8_quant_weights(args["w"], args["B"], args["N"], args["K"], args["w_q"],
                                    args["w_scale"], args["stream"]) == code


def test_quant_weights_zero_rows_is_noop():
    lib = lib_mod.load()
    assert lib.rq_fp8_quant_weights(None, 0, 64, 64, None, None, None) == 0


def test_noalloc_validates_on_the_host():
    """rq_fp8_linear_noalloc rejects bad shapes and requests beyond its static buffer before
    any device query (no GPU here)."""
    lib = lib_mod.load()
    k = 8192
    m = lib_mod.RQ_STATIC_SCRATCH_BYTES // k
    call = lambda m_, k_, n_, act=0: lib.rq_fp8_linear_noalloc(FAKE, m_, k_, act, FAKE, FAKE, n_, FAKE, None)  # noqa: E731
    assert call(m, k, 16) == lib_mod.RQ_ERR_SCRATCH
    assert call(1 << 20, 2048, 16) == lib_mod.RQ_ERR_SCRATCH
    assert call(-1, 64, 16) == RQ_ERR_SHAPE
    assert call(4, 0, 16) == RQ_ERR_SHAPE
    assert call(4, 64, 0) == RQ_ERR_SHAPE
    assert call(0, 64, 16) == 0            # zero rows: a validated no-op
    assert call(0, 24, 16) == RQ_ERR_ALIGN
    assert call(0, 64, 16, act=9) == RQ_ERR_ARG
    assert lib.rq_status_string(lib_mod.RQ_ERR_SCRATCH) == b"request exceeds the static scratch buffer"


def test_topk_validates_on_the_host():
    lib = lib_mod.load()
    call = lambda rows, n, k, ws=FAKE, nb=1 << 30: lib.rq_topk(FAKE, rows, n, k, FAKE, FAKE, ws, nb, None)  # noqa: E731
    assert call(4, 100, 0) == RQ_ERR_SHAPE
    assert call(4, 100, 101) == RQ_ERR_SHAPE
    assert call(4, 5000, 1025) == RQ_ERR_SHAPE
    assert call(-1, 100, 5) == RQ_ERR_SHAPE
    assert call(70000, 100, 5) == RQ_ERR_SHAPE
    assert call(0, 100, 5) == 0                                   # zero rows: a validated no-op
    assert call(4, 100000, 16, ws=None, nb=0) == RQ_ERR_WORKSPACE  # two stages need the workspace
    assert lib.rq_topk_workspace_size(4, 16384, 16) == 0           # one segment: none
    assert lib.rq_topk_workspace_size(32, 262144, 512) == 2 * 32 * 16 * 512 * 8
    assert lib.rq_topk_workspace_size(4, 100, 101) == 0


def test_plan_ready_only_with_permuted_input():
    lib = lib_mod.load()
    ready = lib_mod.RQ_MOE_PLAN_READY
    call = lambda il, T: lib.rq_fp8_moe_grouped_linear(FAKE, il, 0, FAKE, FAKE, T, 2, FAKE, FAKE, 8, 64, 64,  # noqa: E731
                                                       FAKE, 0, FAKE, 1 << 30, None, None)
    assert call(0 | ready, 4) == RQ_ERR_ARG          # token input cannot reuse a plan
    assert call(1 | ready, 0) == 0                   # permuted input: a validated no-op at T = 0
    assert call(2 | ready, 0) == RQ_ERR_ARG          # unknown layout bits stay errors
    # the plan sits first at offsets fixed by (T, top_k, E): the larger call's workspace serves both
    a = lib.rq_fp8_moe_workspace_size(16384, 2, 32, 8192, 2048, 0, 2, 0)
    b = lib.rq_fp8_moe_workspace_size(16384, 2, 32, 2048, 4096, 1, 0, 1)
    assert a > 0 and b > 0


def test_pack_weights_validates_on_the_host():
    lib = lib_mod.load()
    call = lambda b, n, k, src=FAKE, dst=FAKE + 0x1000: lib.rq_fp8_pack_weights(src, b, n, k, dst, None)  # noqa: E731
    assert call(1, 128, 48) == RQ_ERR_ALIGN          # K not a multiple of 64
    assert call(-1, 128, 64) == RQ_ERR_SHAPE
    assert call(1, -1, 64) == RQ_ERR_SHAPE
    assert call(1, 128, 0) == RQ_ERR_SHAPE
    assert call(0, 128, 64) == 0                     # nothing to pack: a validated no-op
    assert call(3, 0, 64) == 0
    assert call(1, 128, 64, src=None) == RQ_ERR_NULL
    assert call(1, 128, 64, dst=FAKE) == RQ_ERR_ARG  # in place is not supported
    assert call(1, 128, 64, dst=FAKE + 8) == RQ_ERR_ALIGN


def test_slab_layout_flag_validates_on_the_host():
    lib = lib_mod.load()
    slabs = lib_mod.RQ_WLAYOUT_SLABS
    lin = lambda m, n, k, g: lib.rq_fp8_linear_ex(FAKE, m, k, 0, 0, FAKE, FAKE, g, n, FAKE, FAKE, 1 << 30,  # noqa: E731
                                                   None, None)
    assert lin(0, 144, 64, slabs) == 0                        # a validated no-op; any N % 16 == 0
    assert lin(0, 128, 80, slabs) == RQ_ERR_ALIGN             # K % 64
    assert lin(0, 144, 80, 0) == 0                            # the row layout takes K % 16 == 0
    assert lin(0, 128, 64, slabs | 3) == RQ_ERR_ARG           # unknown granularity still rejected
    assert lin(0, 128, 64, 0x200) == RQ_ERR_ARG               # unknown layout bits too
    moe = lambda n, k, g: lib.rq_fp8_moe_grouped_linear_ex(FAKE, 0, 0, 0, FAKE, FAKE, 0, 2, FAKE, FAKE, g,  # noqa: E731
                                                            8, n, k, FAKE, 0, FAKE, 1 << 30, None, None)
    assert moe(144, 128, slabs) == 0
    assert moe(256, 96, slabs) == RQ_ERR_ALIGN
