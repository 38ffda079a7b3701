"""ctypes declarations of the C ABI in ``include/rq_fp8.h``.

Loading fails loudly when ``librq_fp8.so`` has not been built: there is no fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librq_fp8.so")

RQ_OK = 0
RQ_ERR_HIP = 6
RQ_ACT_NONE, RQ_ACT_SILU_MUL, RQ_ACT_GATE_SILU = 0, 1, 2
RQ_MOE_IN_TOKENS, RQ_MOE_IN_PERMUTED, RQ_MOE_PLAN_READY = 0, 1, 4
RQ_MOE_OUT_PERMUTED, RQ_MOE_OUT_COMBINED = 0, 1
RQ_KERNEL_QUANT, RQ_KERNEL_GEMM, RQ_KERNEL_COMBINE, RQ_KERNEL_ROUTER, RQ_KERNEL_ATTENTION, RQ_KERNEL_TOPK = \
    0, 1, 2, 3, 4, 5
RQ_WSCALE_CHANNEL, RQ_WSCALE_TENSOR, RQ_WSCALE_BLOCK128 = 0, 1, 2
RQ_WLAYOUT_SLABS = 0x100
RQ_FP8_E4M3, RQ_FP8_E5M2 = 0, 1
RQ_FLAG_EXPERT_ID = 1
RQ_ERR_SCRATCH = 8
RQ_STATIC_SCRATCH_BYTES = 40 << 20

# Every symbol the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t


class DebugOut(ctypes.Structure):
    """``rq_debug_out``: optional device pointers (a_q, a_scale, h)."""
    _fields_ = [("a_q", _P), ("a_scale", _P), ("h", _P)]


SIGNATURES = {
    "rq_fp8_quant_weights": (_I, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "rq_fp8_linear_workspace_size": (_SZ, [_I64, _I64, _I]),
    "rq_fp8_linear_workspace_size_ex": (_SZ, [_I64, _I64, _I64, _I]),
    "rq_fp8_linear": (_I, [_P, _I64, _I64, _I, _P, _P, _I64, _P, _P, _SZ, ctypes.POINTER(DebugOut), _P]),
    "rq_fp8_moe_workspace_size": (_SZ, [_I64, _I, _I64, _I64, _I64, _I, _I, _I]),
    "rq_fp8_moe_grouped_linear": (_I, [_P, _I, _I, _P, _P, _I64, _I, _P, _P, _I64, _I64, _I64,
                                       _P, _I, _P, _SZ, ctypes.POINTER(DebugOut), _P]),
    "rq_fp8_quant_weights_ex": (_I, [_P, _I64, _I64, _I64, _I, _P, _P, _P]),
    "rq_fp8_linear_ex": (_I, [_P, _I64, _I64, _I, _I, _P, _P, _I, _I64, _P, _P, _SZ, ctypes.POINTER(DebugOut),
                              _P]),
    "rq_fp8_moe_grouped_linear_ex": (_I, [_P, _I, _I, _I, _P, _P, _I64, _I, _P, _P, _I, _I64, _I64, _I64,
                                          _P, _I, _P, _SZ, ctypes.POINTER(DebugOut), _P]),
    "rq_moe_router_topk": (_I, [_P, _I64, _I64, _P, _I64, _I, _P, _P, _P, _P]),
    "rq_attention_core": (_I, [_P, _I64, _I, _I, _I, _P, _P]),
    "rq_time_next_kernel": (_I, [_I, _P, _P]),
    "rq_status_string": (ctypes.c_char_p, [_I]),
    "rq_device_supported": (_I, [_I]),
    "rq_debug_flag": (_I, [_I]),
    "rq_topk_workspace_size": (_SZ, [_I64, _I64, _I]),
    "rq_topk": (_I, [_P, _I64, _I64, _I, _P, _P, _P, _SZ, _P]),
    "rq_fp8_linear_noalloc": (_I, [_P, _I64, _I64, _I, _P, _P, _I64, _P, _P]),
    "rq_fp8_pack_weights": (_I, [_P, _I64, _I64, _I64, _P, _P]),
}

_lib = None


class RqError(RuntimeError):
    """A non-zero rq_status returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def load():
    """Load the built library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("librq_fp8.so is not built (expected at %s); run "
                          "fp8_quantized_generative_amd/build.py or __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load().rq_status_string(int(status)).decode()


def check(fn, status):
    if status != RQ_OK:
        raise RqError(fn, status)
