"""C2KV CPU oracle package.  TEST INFRASTRUCTURE ONLY.

Imported solely by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP library
or its binding and imports neither.  Every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle.py`` against values the pages
print, closed forms, invariants, library routines or brute force.

Parity unpinned: none of the functions below.  (The quality of a trained
extractor is out of scope: it needs trained weights and datasets.)
"""
from .c2kv_oracle import *  # noqa: F401,F403
from .c2kv_oracle import (  # noqa: F401
    num_slots, slot_position, extraction_positions, structured_mask, visible_set,
    mask_cell_counts, round_bf16, storage_round, rope_inv_freq, rope_cos_sin,
    rope_rotate, attention, attention_brute, doc_row_offsets, extract_attn,
    compose_positions, compose, append_and_attend, decode_step,
    kv_bytes_per_token, decode_kv_bytes, rms_norm, silu, slot_row_mask, extractor_layer,
)
