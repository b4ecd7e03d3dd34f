"""Pins of the oracle's block-table indexing against the pages' worked examples
and against validation rules.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_block_table_example_blocks_read():
    """'Paged attention' wiki, decode example: which physical blocks hold each
    sequence's cached tokens, and how many tokens each holds."""
    ex = _load("decode_block_table_example.json")
    page, der = ex["stated_by_the_page"], ex["derived_by_definition"]
    table = np.array(page["block_table"], dtype=np.int32)
    bs = page["block_size"]
    assert table.shape == (3, page["max_blocks_per_seq"])
    for s, L in enumerate(page["cache_seqlens"]):
        slots = oracle.token_slots(table[s], L, bs)
        blocks = []
        counts = []
        for b, _ in slots:
            if not blocks or blocks[-1] != b:
                blocks.append(b)
                counts.append(0)
            counts[-1] += 1
        assert blocks == der["physical_blocks_read_for_cached_tokens"][s]
        assert counts == der["tokens_read_per_block"][s]
        # the page's listed blocks are the table's allocated entries, in order
        assert [int(b) for b in table[s] if b != page["unallocated_marker"]] == \
            page["blocks_listed_per_sequence"][s]
        # offsets run 0..BS-1 inside every block, in order
        assert [o for _, o in slots] == [t % bs for t in range(L)]


def test_block_table_example_new_token():
    """Same example: the new token fits in the block already holding the
    cache for sequences 0 and 2, needs the second block for sequence 1."""
    ex = _load("decode_block_table_example.json")
    page, der = ex["stated_by_the_page"], ex["derived_by_definition"]
    table = np.array(page["block_table"], dtype=np.int32)
    bs = page["block_size"]
    for s, L in enumerate(page["cache_seqlens"]):
        slot = oracle.next_slot(table[s], L, bs)
        assert slot == der["new_token_slot"][s]
        last_cached_block = oracle.token_slots(table[s], L, bs)[-1][0]
        fits = (slot // bs) == last_cached_block
        assert fits == page["new_token_fits_in_blocks_already_holding_cache"][s]
        # after the write the token is the last one attended
        after = der["context_lens_after_write"][s]
        assert oracle.token_slots(table[s], after, bs)[-1] == (slot // bs, slot % bs)


def test_decode_walkthrough_example():
    """vLLM paper summary, 'Decoding': 7-token prompt on physical blocks 7, 1;
    step 1 fills the free slot of block 1, step 2 needs physical block 3."""
    ex = _load("decode_walkthrough_example.json")
    der = ex["derived_by_definition"]
    bs = der["block_size"]
    t1 = np.array(der["step1_table"], dtype=np.int32)
    assert oracle.token_slots(t1, 7, bs) == [tuple(x) for x in der["prompt_token_slots"]]
    assert oracle.next_slot(t1, 7, bs) == der["step1_slot"]
    with pytest.raises(ValueError):
        oracle.next_slot(t1, der["step1_context_len_after"], bs)   # block 2 not mapped yet
    t2 = np.array(der["step2_table"], dtype=np.int32)
    assert oracle.next_slot(t2, der["step1_context_len_after"], bs) == der["step2_slot"]
    assert oracle.num_logical_blocks(der["step2_context_len_after"], bs) == 3


def test_num_logical_blocks_brute_force():
    for bs in (1, 4, 16, 32):
        for L in range(0, 200):
            n = 0
            while n * bs < L:
                n += 1
            assert oracle.num_logical_blocks(L, bs) == n


@pytest.mark.parametrize("bad", [
    dict(table=[[2, -1]], lens=[33]),      # -1 inside the context
    dict(table=[[2, 8]], lens=[40]),       # id == num_blocks
    dict(table=[[2, 1]], lens=[65]),       # longer than the table
    dict(table=[[2, 1]], lens=[-1]),       # negative length
])
def test_validate_rejects(bad):
    t = np.array(bad["table"], dtype=np.int32)
    L = np.array(bad["lens"], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.validate(t, L, 32, 8)


def test_validate_ignores_entries_past_the_context():
    t = np.array([[2, -1, 99, -7]], dtype=np.int32)
    oracle.validate(t, np.array([32], dtype=np.int32), 32, 8)
    oracle.validate(t, np.array([0], dtype=np.int32), 32, 8)


def test_validate_head_grouping():
    t = np.array([[0]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.validate(t, np.array([1], dtype=np.int32), 16, 1, num_heads=6, num_kv_heads=4)
