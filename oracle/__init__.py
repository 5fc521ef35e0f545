"""Plain fp64 CPU oracle for paged-KV batch decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library in
``paged_kv_decode_09_amd`` never imports it, links it or calls it, and this
package imports nothing from that library.
"""
from .fp8 import E4M3_TABLE, e4m3_to_f64
from .oracle import (
    widen,
    kv_lengths,
    csr_from_block_table,
    alibi_slopes,
    rope_rotate,
    window_start,
    gather_request,
    attention_state,
    decode_request,
    batch_decode,
    chunk_bounds,
    merge_states,
    decode_request_split,
    batch_decode_split,
    batch_decode_multi,
)

__all__ = [
    "E4M3_TABLE",
    "e4m3_to_f64",
    "widen",
    "kv_lengths",
    "csr_from_block_table",
    "alibi_slopes",
    "rope_rotate",
    "window_start",
    "gather_request",
    "attention_state",
    "decode_request",
    "batch_decode",
    "chunk_bounds",
    "merge_states",
    "decode_request_split",
    "batch_decode_split",
    "batch_decode_multi",
]
