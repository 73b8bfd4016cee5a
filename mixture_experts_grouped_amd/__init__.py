"""MI355X-native routed MoE expert layer with fused rank-r side-LoRA.

The hot path is hand-written HIP for gfx950 behind the C ABI in
include/moelora.h (libmoelora.so, built in-tree by ``build.py``).  This
package adds the ctypes binding (``binding``), the build script and the seeded
synthetic inputs (``inputs``).
"""
from .binding import (  # noqa: F401
    MoeLoraDesc, MoeLoraError, MoeLoraLayer, build_pool, library, make_desc, moe_lora_backward,
    moe_lora_block_m, moe_lora_forward, moe_lora_pool_capacity, moe_lora_workspace_size,
)
