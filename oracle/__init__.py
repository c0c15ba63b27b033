"""CPU oracle of the Ulysses attention front end -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (``head_exchange_amd``) never imports, links or
executes anything here, and this package imports nothing from it: the two share
no code.  The only common module is ``workloads`` (seeded input draws, which hold
none of the method's arithmetic).

Every function is a plain, slow, obviously correct statement of what the pages
define, in float64 for the floating-point steps.  See ``qkvx_oracle`` for the
functions and the passages each follows.  Parity status: every function here is
pinned by a CPU test in ``tests/test_oracle_pins.py`` against something other
than itself (exact brute-force sums, closed forms, invariants, library routines,
the pages' printed schedule example).
"""
from .qkvx_oracle import (  # noqa: F401
    EPS, bf16_bits_to_f64, f64_to_bf16_rne, qkv_projection, rmsnorm_heads,
    rope_rotate_half, rope_interleaved, front_end_values, front_end_rows,
    receive_slots, scatter_heads, pack_qkv_head_chunk_payload,
    pack_qkv_head_chunk_into, merge_output_head_chunk, POISON_BITS,
    gather_heads, exchange_chunks, pack_output_sequence_chunk_payload,
    pack_output_sequence_chunk_into, gather_output_head_chunk,
)
