"""CPU oracle for the hybrid-batch decoder layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
or call this package.  The product path (the HIP library and its Python binding) never does, and this
package imports nothing from it.
"""
from .multi import apply_multi_rows, layer_forward_multi, multi_positions
from .paged import apply_paged_rows, gather_cache, layer_forward_paged, paged_slot
from .layer import (apply_new_rows, apply_stack_rows, attend_rows, chunk_mask, gelu, layer_forward,
                    layer_norm, positions, rms_norm, rope_inv_freq, rope_rotate, silu, stack_forward)

__all__ = ["apply_multi_rows", "apply_new_rows", "apply_paged_rows", "gather_cache", "layer_forward_paged",
           "paged_slot", "apply_stack_rows", "attend_rows", "chunk_mask", "gelu",
           "layer_forward", "layer_forward_multi", "layer_norm", "multi_positions", "positions", "rms_norm",
           "rope_inv_freq", "rope_rotate", "silu", "stack_forward"]
