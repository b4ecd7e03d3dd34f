"""Pins of the oracle's block copy (copy-on-write, swap), CPU only."""
import numpy as np
import pytest

import oracle


def _pools(rng, NB, KVH=2, BS=16, D=8, dt=np.float16):
    k = rng.normal(0, 1, (NB, KVH, BS, D)).astype(dt)
    v = rng.normal(0, 1, (NB, KVH, BS // 4, D, 4)).astype(dt)
    return k, v


def test_copy_by_hand():
    """Block 3 becomes block 1 and block 2 becomes block 0, element by
    element over every kv head of K and V; nothing else changes and the
    inputs are not modified."""
    rng = np.random.default_rng(0)
    k, v = _pools(rng, 5)
    k0, v0 = k.copy(), v.copy()
    m = np.array([[1, 3], [0, 2]], dtype=np.int32)
    nk, nv = oracle.copy_blocks(k, v, k, v, m)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)
    for b in range(5):
        want = {3: 1, 2: 0}.get(b, b)
        for h in range(2):
            for t in range(16):
                for d in range(8):
                    assert nk[b, h, t, d] == k0[want, h, t, d]
                    assert nv[b, h, t // 4, d, t % 4] == v0[want, h, t // 4, d, t % 4]


def test_copy_between_pools_and_skips():
    """Swap-out shape: a 4-block source pool into a 6-block destination pool;
    pairs with a negative or out-of-range id are skipped; fp8 codes are
    bytes."""
    rng = np.random.default_rng(1)
    sk = rng.integers(0, 256, (4, 2, 16, 8), dtype=np.uint8)
    sv = rng.integers(0, 256, (4, 2, 4, 8, 4), dtype=np.uint8)
    dk = np.zeros((6, 2, 16, 8), dtype=np.uint8)
    dv = np.zeros((6, 2, 4, 8, 4), dtype=np.uint8)
    m = np.array([[2, 5], [-1, 0], [4, 1], [0, 6], [3, 0]], dtype=np.int32)
    nk, nv = oracle.copy_blocks(sk, sv, dk, dv, m)
    assert np.array_equal(nk[5], sk[2]) and np.array_equal(nv[5], sv[2])
    assert np.array_equal(nk[0], sk[3]) and np.array_equal(nv[0], sv[3])
    for b in (1, 2, 3, 4):
        assert not nk[b].any() and not nv[b].any()


def test_copy_rejects_conflicts():
    rng = np.random.default_rng(2)
    k, v = _pools(rng, 4)
    with pytest.raises(ValueError):
        oracle.copy_blocks(k, v, k, v, np.array([[0, 2], [1, 2]], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.copy_blocks(k, v, k, v, np.array([[0, 1], [1, 3]], dtype=np.int32))


def test_cow_then_write_keeps_the_other_sequence_and_gives_the_writer_its_token():
    """Parallel sampling ("How does paged attention work (in detail)",
    section 3.3): A and B share a 20-token prompt in physical blocks [2, 5]
    (block 5 half full).  B's next token would land in shared block 5, so
    block 5 is copied to a free block and B's entry re-pointed before the
    write.  A's attention is unchanged; B attends over the prompt and its own
    token, gathered by hand."""
    rng = np.random.default_rng(3)
    BS, KVH, D, NB = 16, 2, 8, 8
    k, v = _pools(rng, NB, KVH, BS, D)
    table = np.array([[2, 5], [2, 5]], dtype=np.int32)
    L = np.array([20, 20], dtype=np.int32)
    refs = {2: 2, 5: 2}
    free = [7, 0, 1]
    q = rng.normal(0, 1, (2, KVH, D)).astype(np.float16)
    before = oracle.paged_decode(q, k, v, table, L, 0.4, KVH, BS, "f16", "f16")

    pair, row_b = oracle.cow_step(table[1], 20, BS, refs, free)
    assert pair == (5, 7) and row_b == [2, 7] and refs == {2: 2, 5: 1, 7: 1} and free == [0, 1]
    assert oracle.cow_step(table[0], 20, BS, refs, free) == (None, [2, 5])   # now private
    k1, v1 = oracle.copy_blocks(k, v, k, v, np.array([pair], dtype=np.int32))
    table2 = np.array([table[0], row_b], dtype=np.int32)
    nk = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    nv = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    slot = oracle.next_slot(table2[1], 20, BS)
    assert slot == 7 * BS + 4
    k2, v2 = oracle.cache_write(nk, nv, k1, v1, np.array([slot], dtype=np.int32), BS, "f16")

    after = oracle.paged_decode(q, k2, v2, table2, np.array([20, 21], dtype=np.int32), 0.4, KVH,
                                BS, "f16", "f16")
    assert np.array_equal(after[0], before[0])
    assert np.array_equal(k2[5], k[5]) and np.array_equal(v2[5], v[5])
    for h in range(KVH):
        rows_k = [k[table[0, t // BS], h, t % BS] for t in range(20)] + [nk[0, h]]
        rows_v = [v[table[0, t // BS], h, (t % BS) // 4, :, t % 4] for t in range(20)] + [nv[0, h]]
        K = np.array(rows_k, dtype=np.float64)
        V = np.array(rows_v, dtype=np.float64)
        x = float(np.float32(0.4)) * (K @ q[1, h].astype(np.float64))
        w = np.exp(x - x.max())
        np.testing.assert_allclose(after[1, h], (w / w.sum()) @ V, rtol=1e-12, atol=1e-14)


def test_swap_out_and_back_in_restores_the_attention():
    """Preemption by swapping (same page, section 4.3; vLLM paper summary,
    section 5): a sequence's blocks go to a CPU pool, their GPU blocks are
    reused by others, then the blocks come back into other free GPU blocks
    and the table is re-pointed: the attention is bit-identical."""
    rng = np.random.default_rng(4)
    BS, KVH, D = 16, 2, 8
    k, v = _pools(rng, 10, KVH, BS, D)
    row = np.array([[6, 1, 8]], dtype=np.int32)
    L = np.array([40], dtype=np.int32)
    q = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    before = oracle.paged_decode(q, k, v, row, L, 0.3, KVH, BS, "f16", "f16")
    ck = np.zeros((3, KVH, BS, D), dtype=np.float16)
    cv = np.zeros((3, KVH, BS // 4, D, 4), dtype=np.float16)
    ck, cv = oracle.copy_blocks(k, v, ck, cv, np.array([[6, 0], [1, 1], [8, 2]], dtype=np.int32))
    k[[6, 1, 8]] = np.float16(np.nan)                 # reused by other sequences meanwhile
    v[[6, 1, 8]] = np.float16(np.nan)
    k, v = oracle.copy_blocks(ck, cv, k, v, np.array([[0, 3], [1, 9], [2, 0]], dtype=np.int32))
    after = oracle.paged_decode(q, k, v, np.array([[3, 9, 0]], dtype=np.int32), L, 0.3, KVH, BS,
                                "f16", "f16")
    assert np.array_equal(after, before)
