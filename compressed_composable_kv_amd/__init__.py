"""C2KV hot path on AMD Instinct MI355X (gfx950).

Python binding of libc2kv.so: structured-flow extraction attention,
RoPE-realigned composition of compressed slot caches, and GQA prefill /
decode over the composed cache.  See include/c2kv.h for the C ABI.
"""
from .ops import (  # noqa: F401
    C2KVError, attn_decode, attn_decode_noalloc, attn_prefill, compose, compose_staged, extract_attn, extract_layer, gate_up_interleave, host_device_ptr, mask_cells, tile_schedule,
    num_slots, packed_rows, rope_inv_freq, slot_position, slot_views, version,
    workspace_size_decode, workspace_size_extract, workspace_size_extract_layer, workspace_size_prefill,
)
