"""CPU oracle for the MoE expert-LoRA fold (test infrastructure only).

This package is a plain, slow, obviously correct restatement of what the
fold and its host-side integer work compute, written from the pages that
describe the method:

* "moe_row_adapter.rs" (the GPU-free MoE LoRA routing module): the per-request
  fold decision, the decode-batch refusal and the two per-row adapter maps;
* "moe_lora_grouped" (the launcher module index): table packing, the window
  split and its tile count, the row-to-token rule, the skip invariant and the
  two fold formulas (gather over flat decode rows, grouped over expert-sorted
  prefill rows).

Floating point is fp64 throughout; bf16 inputs are widened exactly. Nothing
here is blocked, fused or reordered beyond the definitions.

Only the test suite, the smoke check of the package entry file and the CPU
baseline leg of the benchmark may import this package. The device library
never imports, links or calls it, and this package never imports the device
library. Its only shared dependency is the seeded input generator module,
which holds none of the fold's arithmetic.
"""
from .host import (  # noqa: F401
    FOLD,
    SKIP,
    REFUSE,
    RefuseError,
    resolve_moe_lora_route,
    ensure_decode_route_servable,
    build_moe_row_adapter_host,
    build_moe_row_adapter_decode,
    pack_expert_tables,
    grouped_down_windows,
    grouped_down_wc,
    gather_row_token,
    MAX_EXPERT_ID,
)
from .multi import (  # noqa: F401
    resolve_moe_lora_route_multi,
    build_moe_row_adapter_decode_multi,
    pack_expert_tables_multi,
    fold_gather_multi,
)
from .fold import (  # noqa: F401
    bf16_to_f64,
    fold_gather_scalar,
    fold_gather,
    fold_grouped_scalar,
    fold_grouped,
    fold_grouped_windows,
)
