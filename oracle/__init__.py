"""CPU oracle for paged decode attention, the KV cache write and whole-block
copies (copy-on-write, swapping).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import anything from this package.  The GPU library never calls
it, shares no code with it, and must fail loudly when its HIP build is
missing instead of falling back to this.

Everything here is plain numpy in fp64 (the fp8 quantiser takes its rounding
decision on a binary32 product, the precision the cache writer uses), written
to be checked by eye against the pages it cites.  It is pinned, independently
of itself, by tests/test_oracle_*.py: the worked block-table examples of the
pages, brute force on tiny inputs, scaled_dot_product_attention as a library
special case, closed forms (one token, constant V, two tokens, q = 0, a
needle), invariances (relabelled physical blocks, another block size,
partition count), an exhaustive check of the e4m3fn codec, and for the block
copies a hand-checked copy plus copy-on-write and swap scenarios whose
attention is known.  No function
here is "parity unpinned".
"""
from .block_manager import BlockManager, NoFreeBlocks  # noqa: F401
from .block_ops import copy_blocks, cow_step  # noqa: F401
from .formats import (  # noqa: F401
    E4M3_MAX,
    bf16_to_f64,
    e4m3fn_encode,
    e4m3fn_round,
    e4m3fn_to_f64,
    f16_to_f64,
    inv_scale_f32,
    quantise_e4m3fn,
    to_f64,
)
from .paged_attention import (  # noqa: F401
    cache_write,
    decode_append,
    decode_sequence,
    merge_partials,
    next_slot,
    num_logical_blocks,
    paged_decode,
    paged_decode_partitioned,
    paged_prefill,
    partition_partials,
    request_index,
    softmax_stats,
    stored_rows,
    token_slots,
    v_tiles_to_rows,
    validate,
)
