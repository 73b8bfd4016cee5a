"""CPU oracle for the routed MoE expert layer with rank-r side-LoRA.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``mixture_experts_grouped_amd``) never imports it,
and this package imports nothing from the product path.

The oracle is plain, slow and written to be checked against the pages by eye:
numpy in float64 on the exact values of the bf16 inputs, one Python loop over
experts, no fusion and no algebraic regrouping beyond what the definition
states.  Its pins (closed forms, finite differences, identities, brute force
on tiny inputs) live in ``tests/test_oracle_*.py``.

Modules:
  pool     -- expert-contiguous pool padded per expert (integer metadata)
  moe_lora -- forward and backward of the layer, per route
  mxfp4    -- exact dequantisation of e2m1 values with e8m0 block scales
  multi_adapter -- several adapters in one pass, one root of tokens each
"""
from . import pool, moe_lora, mxfp4, multi_adapter  # noqa: F401
