"""CPU oracle for batch-1 / small-M decode through quantized MoE expert weights.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``quantized_moe_weight_amd`` and its HIP library) never imports, links or calls
anything here, and this package imports nothing from the product path.  The two
share no code; the only common module is ``workloads`` (seeded random inputs,
none of the method's arithmetic).

The oracle is written to be plain and obviously correct, not fast: numpy in
float64, exact codec tables built from the format definitions, a
dequantise-then-fp64-matmul for every linear layer.  Each function cites the
passage of the source pages it follows.  Source pages are cited by handle:

* [Sionic]  Sionic AI blog, "GPU 커널부터 새로 짜서 GLM-5.2 속도 10배 올리기"
            (rewriting the GPU kernels to make GLM-5.2 ten times faster).
            Sections: intro (bandwidth roofline), 1 low SM occupancy,
            2 pipeline serialisation, 3 register pressure, 4 too many small
            kernels, 5 MTP (with the per-token traffic table), 7 MTP caveats,
            8c kernel-level optimisation.
* [M3]      aiwitness community post, "GLM 5.3 Flash Q4 @ 60tps / 550tps on
            M3 Ultra".
* [CMP]     aiwitness community post, "CMP 170HX 64GB 2개: GLM-5.3-Flash 384K
            컨텍스트 / ~90 tok/s (EXL3, HBM 우선 설정) 및 Qwen3.8 비교".
* [M1]      rbeckner.com, "Qwen 3.8-27B M1 Ultra에서: 12.1에서 20.3 tok/s까지
            모든 것을 측정하여".

Where the pages leave a step open (the FP8 variant, the scale rule, rounding,
the int4 layout, the SiLU layout ...) the oracle takes the plainest reading and
says so in the docstring of the function concerned.

Parity status: every public function here is pinned by ``tests/test_oracle_*``
against values that do not come from this package (an independent library
conversion, exact rational brute force, closed forms printed on the pages,
invariants).  No function is "parity unpinned".
"""
from .codecs import (E4M3_MAX, e4m3_decode, e4m3_encode, bf16_round, bf16_bits,
                     bf16_bits_to_f64, q4_pack, q4_unpack)
from .quant import block_quant_fp8, act_quant_fp8, dequant_fp8, q4_quant, dequant_q4
from .linear import gemv_fp8, silu_mul, gemv_q4
from .moe import route_topk, router_logits, moe_layer, union_of_experts
from . import traffic

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "bf16_round", "bf16_bits", "bf16_bits_to_f64",
    "q4_pack", "q4_unpack", "block_quant_fp8", "act_quant_fp8", "dequant_fp8", "q4_quant",
    "dequant_q4", "gemv_fp8", "silu_mul", "gemv_q4", "route_topk", "moe_layer",
    "union_of_experts", "traffic",
]
