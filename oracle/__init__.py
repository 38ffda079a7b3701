"""Plain, slow CPU oracle for the W8A8 FP8 linear of OneRec-V2 post-training-quantized serving.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this package: only the tests, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table or
constant generator with the HIP library under ``fp8_quantized_generative_amd``.

What it computes, and where the pages fix it:

* page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈",
  section 关键证据: weights are quantized offline per output channel, activations
  per token at run time, the product runs in FP8 with FP32 accumulation, and the
  result is cast back to FP16 before the next layer; only the attention q/k/v/o
  linears, the dense FFN linears and the MoE grouped GEMM are quantized.
* page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §1.2 (the FP8 range is
  +/-448, i.e. OCP E4M3), §2.2 (the per-token quantizer: an amax-derived scale
  with an epsilon clamp, rounding and clamping) and §2.3 / Fig. 2 (FP16 input,
  dynamic quantization, FP8 GEMM, dequantization, FP16 output).

Arithmetic is float64 and integers.  Every rounding is explicit.  Modules:

* ``e4m3``   - OCP OFP8 E4M3 decode table and saturating round-to-nearest-even encode.
* ``e5m2``   - the same for OCP OFP8 E5M2 (activations in E5M2: page "FP8量化在生成式推荐系统
               OneRec-V2中的优化实践", §2.2).
* ``quant``  - the row quantizer (per output channel for weights, per token for activations).
* ``linear`` - exact FP8 dot products, per-token x per-channel dequantization to FP16, and
               the parity tolerance.
* ``ffn``    - the SiLU(gate) * up intermediate of the dense and expert FFNs.
* ``moe``    - the MoE routing plan, grouped linear over experts and the weighted combine.
* ``attention`` - the FP16 short-context attention core between the QKV and O linears.
* ``router`` - the FP16 MoE gate: logits, top-k expert selection and combine weights.
* ``wscale`` - weight scales per tensor and per 128 x 128 block (page "FP8量化在生成式推荐
               系统OneRec-V2中的优化实践", §2.1 / §2.2) and the linear that uses them.
* ``topk``   - batched top-k of FP16 candidate rows for beam search (the RadixSelect TopK of
               page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §3.2).
* ``layout`` - the slab byte layout of quantized weights (this library's own layout; the
               pages fix none): a permutation of bytes, no arithmetic.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against
values fixed independently of this code (the OCP format definition, closed forms,
brute force over exact rationals, PyTorch's own float8_e4m3fn conversion and SiLU).
No function is "parity unpinned".
"""

from . import attention, e4m3, e5m2, quant, linear, ffn, moe, router, topk, wscale, layout  # noqa: F401

__all__ = ["attention", "e4m3", "e5m2", "quant", "linear", "ffn", "moe", "router", "topk", "wscale"]
