"""Paged decode attention for MI355X (gfx950): a C-ABI HIP library and its
Python binding.  See include/pa.h for the ABI."""
from .binding import (  # noqa: F401
    EXPORTS,
    BlockManager,
    PagedAttentionError,
    cache_write,
    copy_blocks,
    decode,
    decode_append,
    decode_partitioned,
    decode_partitioned_noalloc,
    decode_partitioned_only,
    lib,
    partition_workspace,
    prefill,
    reduce,
)
