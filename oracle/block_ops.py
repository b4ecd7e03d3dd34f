"""Whole-block operations on a block pool: copy-on-write and swapping.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

A physical block holds the K/V of block_size tokens for every kv head
("How does paged attention work (in detail)", section 3.1).  Sequences that
share a prefix point at the same physical blocks; before one of them writes
into a shared block, the block is copied and that sequence's table entry is
re-pointed to the copy (same page, section 3.3).  A preempted sequence's
blocks are moved to CPU memory and brought back when it is rescheduled
(same page, section 4.3; vLLM paper summary, section 5).  Both are the same
operation on the pools: block dst of the destination pool becomes a copy of
block src of the source pool.
"""
from __future__ import annotations

import numpy as np


def copy_blocks(src_k, src_v, dst_k, dst_v, mapping):
    """New destination pools (copies of dst_k/dst_v) in which block m[i, 1]
    holds the bytes of source block m[i, 0], for every pair with both ids in
    range; other pairs are skipped.  The sources are read as they were before
    the call.  A destination listed twice, or a block that is both a source
    and a destination when the pools are the same, is rejected."""
    src_k, src_v = np.asarray(src_k), np.asarray(src_v)
    out_k, out_v = np.array(dst_k, copy=True), np.array(dst_v, copy=True)
    pairs = [(int(s), int(d)) for s, d in np.asarray(mapping).reshape(-1, 2).tolist()]
    valid = [(s, d) for s, d in pairs
             if 0 <= s < src_k.shape[0] and 0 <= d < out_k.shape[0]]
    dsts = [d for _, d in valid]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block is written twice")
    if dst_k is src_k and set(dsts) & {s for s, _ in valid}:
        raise ValueError("a block is both a source and a destination")
    for s, d in valid:
        out_k[d] = src_k[s]
        out_v[d] = src_v[s]
    return out_k, out_v


def cow_step(table_row, context_len: int, block_size: int, ref_counts: dict, free_list: list):
    """Copy-on-write before writing the token at position context_len.

    If the physical block that position falls in is shared (reference count
    > 1), take a free block, return the copy pair (src, dst) and the row with
    the entry re-pointed; the shared block loses one reference and the new
    one has one.  Otherwise return (None, row unchanged)."""
    row = list(table_row)
    j = int(context_len) // block_size
    b = int(row[j])
    if ref_counts.get(b, 0) <= 1:
        return None, row
    if not free_list:
        raise MemoryError("no free block for the copy")
    nb = free_list.pop(0)
    ref_counts[b] -= 1
    ref_counts[nb] = 1
    row[j] = nb
    return (b, nb), row
