"""The seeded generators: determinism and block-table structure (CPU only)."""
import numpy as np
import torch

import oracle
import workloads


def _check_tables(wl):
    table = wl.block_table.cpu().numpy()
    L = wl.context_lens.cpu().numpy()
    BS = wl.block_size
    owners = {}
    shared = set(wl.shared_blocks)
    for s in range(wl.num_seqs):
        n = oracle.num_logical_blocks(int(L[s]) + 1, BS)     # room for the new token
        row = table[s]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < wl.num_blocks)
        assert np.all(row[n:] == -1)
        for b in row[:n]:
            if int(b) in shared:
                continue
            assert int(b) not in owners, "private block used twice"
            owners[int(b)] = s
        assert int(wl.slot_mapping[s]) == oracle.next_slot(row, int(L[s]), BS)
    oracle.validate(table, L + 1, BS, wl.num_blocks, wl.num_heads, wl.num_kv_heads)


def test_worked_example_is_the_pages_table():
    wl = workloads.worked_example()
    assert wl.block_table.tolist() == [[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]]
    assert wl.context_lens.tolist() == [30, 32, 70]
    assert wl.slot_mapping.tolist() == [94, 32, 198]
    assert tuple(wl.q.shape) == (3, 4, 64) and tuple(wl.k_cache.shape) == (8, 4, 32, 64)
    assert tuple(wl.v_cache.shape) == (8, 4, 8, 64, 4)
    _check_tables(wl)


def test_small_variants_structure_and_determinism():
    a = workloads.llama7b_mha(num_seqs=5, len_range=(1, 70))
    b = workloads.llama7b_mha(num_seqs=5, len_range=(1, 70))
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.block_table, b.block_table)
    _check_tables(a)
    _check_tables(workloads.gqa(num_seqs=4, len_range=(16, 80)))
    _check_tables(workloads.long_context(num_seqs=2, len_range=(600, 1500), num_heads=2))


def test_fp8_shared_prefix_structure():
    wl = workloads.fp8_shared_prefix(num_seqs=16, cap=700, num_heads=8, num_kv_heads=2,
                                     prefix_tokens=64)
    _check_tables(wl)
    table = wl.block_table.numpy()
    L = wl.context_lens.numpy()
    pre = list(wl.shared_blocks)
    assert len(pre) == 4
    sharing = [s for s in range(16) if list(table[s, :4]) == pre]
    assert len(sharing) == 4 and all(L[s] >= 64 for s in sharing)
    assert wl.k_cache.dtype == torch.float8_e4m3fn
    codes = wl.k_cache.view(torch.uint8)
    assert not bool(((codes & 0x7F) == 0x7F).any())            # no NaN codes
    assert wl.k_scale > 0 and wl.v_scale > 0
