"""CPU oracle for the fused cascaded reductions: TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The library's product path never calls it, and it
shares no code with the HIP kernels or their host layer.

Everything here is plain numpy in float64 on the exact input values the GPU
sees (fp32, or bf16 upcast losslessly). Where the fused incremental method
reaches a result that has a plain definition (attention, its multi-segment
split and merge, the MoE gate), the oracle is that plain multi-pass definition,
not the fused loop. The quantised GEMM's codes and scales are also defined
literally (absmax, then scale, then round), because rounding has no incremental
form.

Sources (the pages describe one paper, "RedFuser: An Automatic Operator Fusion
Framework for Cascaded Reductions on AI Accelerators", ASPLOS 2026):

* [abstract]  the paper's abstract page;
* [explainer] "RedFuser框架：AI加速器中的算子融合技术解析" (a Chinese explainer
  with pseudocode in its sections 2.2, 2.3, 4.1, 4.2 and 4.3);
* [summary]   the Dutch technical summary "RedFuser: An Automatic Operator Fusion
  Framework for Cascaded Reductions on AI Accelerators", section
  "Technische samenvatting" -> "Methodologie" items 1-3.

Every function is pinned by tests that do not re-type its formula (brute force
on tiny inputs, closed forms, invariants, library cross-checks, exhaustive
codec checks); no function is "parity unpinned".
"""
from .attention import attention, attention_incremental, decode, decode_streaming, mla_decode
from .segments import segment_bounds, split_partials, merge_partials, decode_split_merge
from .moe import moe_route, gate_scores, topk_softmax
from . import cascade
from .quant import (E4M3_MAX, e4m3fn_decode, e4m3fn_encode, fl32, quantize_rows,
                    quant_gemm, quant_gemm_acc)

__all__ = [
    "attention", "attention_incremental", "decode", "decode_streaming", "mla_decode",
    "segment_bounds", "split_partials", "merge_partials", "decode_split_merge",
    "moe_route", "gate_scores", "topk_softmax", "cascade",
    "E4M3_MAX", "e4m3fn_decode", "e4m3fn_encode", "fl32", "quantize_rows",
    "quant_gemm", "quant_gemm_acc",
]
