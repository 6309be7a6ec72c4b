"""CPU oracle for the fused grouped W4A16 MoE expert layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct definition of what the layer computes, written from
"Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference" (abstract;
Fig. 1 caption; Tab. 1) plus the readings listed in each function's docstring.
Floating point is carried in fp64 except where a step rounds to a stored type
(bf16 logits, bf16 scales, fp32 routing weights).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its binding) never does, and this
package imports nothing from it.

Parity pins: every function is pinned by a CPU test against closed forms, brute force
or exact arithmetic. Parity unpinned: absolute layer-output values (no page prints a
tensor) and the choice of scale divisor absmax/7 (a reading, not a page fact).
"""
from .quant import quantize_group128, dequantize_group128, bf16_bits_to_f64, f64_to_bf16_bits
from .layout import (packed_expert_bytes, pack_expert, unpack_expert, TILE_ROWS, GROUP, bf16_expert_bytes,
                     pack_expert_bf16)
from .router import router_logits, topk_ids, topk_weights
from .group import group_tokens
from .moe import (QuantExpert, DenseExpert, quantize_expert, expert_mlp, forward_per_token,
                  forward_grouped, combine, moe_layer, knockout_rows)
from .lru import LRUSlotCacheSim

__all__ = [
    "quantize_group128", "dequantize_group128", "bf16_bits_to_f64", "f64_to_bf16_bits",
    "packed_expert_bytes", "pack_expert", "unpack_expert", "TILE_ROWS", "GROUP", "bf16_expert_bytes",
    "pack_expert_bf16", "DenseExpert",
    "router_logits", "topk_ids", "topk_weights", "group_tokens",
    "QuantExpert", "quantize_expert", "expert_mlp", "forward_per_token", "forward_grouped",
    "combine", "moe_layer", "knockout_rows", "LRUSlotCacheSim",
]
