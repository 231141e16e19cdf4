"""CPU float64 oracle for block-paged KV attention.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the library
(``block_paged_kv_append_amd``) never does and shares no code with it.
"""
from .paged_attention import (  # noqa: F401
    BLOCK,
    append,
    attend,
    column_mass,
    copy_blocks,
    decode,
    decode_append,
    decode_splitk,
    gather_sequence,
    merge_partials,
    new_token_slots,
    prefill,
    scores,
    values,
    visible,
)
