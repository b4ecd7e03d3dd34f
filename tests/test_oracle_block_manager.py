"""Pins of the oracle's host block manager (CPU only)."""
import json
import os
import random

import numpy as np
import pytest

import oracle
from oracle import BlockManager, NoFreeBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_paper_summary_decode_walkthrough():
    """vLLM paper summary, section 3: a 7-token prompt in blocks 7 and 1
    (block size 4); the first decode token takes the free slot of block 1,
    the second needs a new block, 3."""
    ex = _load("decode_walkthrough_example.json")
    d = ex["derived_by_definition"]
    BS = d["block_size"]
    order = [7, 1, 3, 0, 2, 4, 5, 6]
    bm = BlockManager(8, 0, BS, gpu_free_order=order)
    bm.add_sequence("p", ex["stated_by_the_page"]["prompt_tokens"])
    assert bm.table("p") == [7, 1]
    slot, pair = bm.append_slot("p")
    assert (slot, pair) == (d["step1_slot"], None) and bm.length("p") == d["step1_context_len_after"]
    assert bm.table("p") + [-1] == d["step1_table"]
    slot, pair = bm.append_slot("p")
    assert (slot, pair) == (d["step2_slot"], None) and bm.table("p") == d["step2_table"]
    assert bm.length("p") == d["step2_context_len_after"]


def test_batching_wiki_decode_example():
    """The wiki's decode batch (block size 32, cached 30, 32, 70 tokens):
    the new tokens go to slots 94, 32, 198 and only sequence 1 needs a
    second block, giving the page's table [[2], [0, 1], [3, 5, 6]]."""
    ex = _load("decode_block_table_example.json")
    page, d = ex["stated_by_the_page"], ex["derived_by_definition"]
    bm = BlockManager(8, 0, page["block_size"], gpu_free_order=[2, 0, 3, 5, 6, 1, 4, 7])
    for sid, L in enumerate(page["cache_seqlens"]):
        bm.add_sequence(sid, L)
    slots = [bm.append_slot(sid)[0] for sid in range(3)]
    assert slots == d["new_token_slot"]
    assert [bm.table(s) for s in range(3)] == page["blocks_listed_per_sequence"]
    assert [bm.length(s) for s in range(3)] == d["context_lens_after_write"]


def test_allocation_from_the_front_and_release_to_the_back():
    """How-it-works, section 3.2: blocks come from the head of the free
    queue with one reference; freeing drops the count and returns blocks
    whose count reaches zero."""
    bm = BlockManager(10, 0, 16)
    bm.add_sequence("a", 40)                 # 3 blocks
    bm.add_sequence("b", 17)                 # 2 blocks
    assert bm.table("a") == [0, 1, 2] and bm.table("b") == [3, 4]
    bm.free("a")
    assert bm.gpu.free == [5, 6, 7, 8, 9, 0, 1, 2]
    bm.add_sequence("c", 64)
    assert bm.table("c") == [5, 6, 7, 8]
    with pytest.raises(NoFreeBlocks):
        bm.add_sequence("d", 65)             # 5 blocks, 4 free: nothing changes
    assert "d" not in bm.seqs and bm.num_free() == 4


def test_fork_shares_and_copy_on_write_splits():
    """Parallel sampling (how-it-works, section 3.3): after a fork both
    sequences reference the same blocks; the first write into the shared
    last block gives the writer a copy; the other then writes in place."""
    bm = BlockManager(6, 0, 4)
    bm.add_sequence("a", 6)                  # blocks [0, 1], block 1 half full
    bm.fork("a", "b")
    assert bm.ref_count(0) == 2 and bm.ref_count(1) == 2
    slot, pair = bm.append_slot("b")
    assert pair == (1, 2) and bm.table("b") == [0, 2] and slot == 2 * 4 + 2
    assert bm.ref_count(1) == 1 and bm.ref_count(2) == 1 and bm.ref_count(0) == 2
    slot, pair = bm.append_slot("a")
    assert pair is None and slot == 1 * 4 + 2
    # the same decision as the block-op oracle's copy-on-write step
    refs = {0: 2, 1: 2}
    p2, row = oracle.cow_step([0, 1], 6, 4, refs, [2])
    assert p2 == (1, 2) and row == [0, 2]


def test_swap_out_and_in():
    """How-it-works, section 4.3 and the paper summary, section 5: a
    sequence's blocks move to the CPU pool (its GPU blocks are freed, a
    shared one stays for its other user) and come back into free GPU
    blocks; the copies to perform are returned in table order."""
    bm = BlockManager(8, 4, 4)
    bm.add_sequence("a", 9)                  # [0, 1, 2]
    bm.fork("a", "b")
    bm.add_sequence("c", 4)                  # [3]
    pairs = bm.swap_out("a")
    assert pairs == [(0, 0), (1, 1), (2, 2)] and bm.table("a") == [0, 1, 2]
    assert bm.ref_count(0) == 1 and bm.num_free(True) == 4 and bm.num_free(False) == 1
    bm.free("b")                             # the shared blocks return now
    assert bm.gpu.free == [4, 5, 6, 7, 0, 1, 2]
    back = bm.swap_in("a")
    assert back == [(0, 4), (1, 5), (2, 6)] and bm.table("a") == [4, 5, 6]
    assert bm.num_free(False) == 4 and bm.length("a") == 9
    with pytest.raises(NoFreeBlocks):
        BlockManager(2, 1, 4).add_sequence("x", 12)


def test_random_traces_keep_the_invariants():
    """Random operation traces: every block is either free or referenced
    exactly as often as tables list it; a table has ceil(len / BS) blocks;
    slots handed out are distinct and lie in the sequence's own blocks."""
    rng = random.Random(0)
    for trial in range(20):
        NG, NC, BS = 40, 20, rng.choice([1, 4, 16])
        bm = BlockManager(NG, NC, BS)
        live, next_id, written = [], 0, {}
        for _ in range(300):
            op = rng.random()
            try:
                if op < 0.25 or not live:
                    bm.add_sequence(next_id, rng.randint(0, 3 * BS))
                    live.append(next_id)
                    next_id += 1
                elif op < 0.35:
                    bm.fork(rng.choice([s for s in live if bm.seqs[s]["on_gpu"]] or [None]),
                            next_id)
                    live.append(next_id)
                    next_id += 1
                elif op < 0.75:
                    s = rng.choice(live)
                    if bm.seqs[s]["on_gpu"]:
                        slot, pair = bm.append_slot(s)
                        assert slot // BS in bm.table(s)
                elif op < 0.85:
                    s = rng.choice(live)
                    bm.free(s)
                    live.remove(s)
                elif op < 0.93:
                    s = rng.choice(live)
                    if bm.seqs[s]["on_gpu"]:
                        bm.swap_out(s)
                else:
                    s = rng.choice(live)
                    if not bm.seqs[s]["on_gpu"]:
                        bm.swap_in(s)
            except (NoFreeBlocks, KeyError):
                pass
            for pool, on_gpu, n in ((bm.gpu, True, NG), (bm.cpu, False, NC)):
                counts = {}
                for st in bm.seqs.values():
                    if st["on_gpu"] == on_gpu:
                        for b in st["blocks"]:
                            counts[b] = counts.get(b, 0) + 1
                assert counts == pool.refs
                assert sorted(pool.free + list(pool.refs)) == list(range(n))
            for st in bm.seqs.values():
                assert len(st["blocks"]) == -(-st["len"] // BS)
