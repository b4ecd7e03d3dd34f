"""Pins of the oracle's cache write (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    with open(os.path.join(GOLDEN, "decode_block_table_example.json")) as f:
        return json.load(f)


def test_block_table_example_write_touches_exactly_the_new_slots():
    """'Paged attention' wiki decode example: the step's three new tokens go
    to slots 94, 32, 198 of the 8-block pool; nothing else changes."""
    ex = _example()
    BS, KVH, D, NB = ex["stated_by_the_page"]["block_size"], 4, 64, 8
    slots = np.array(ex["derived_by_definition"]["new_token_slot"], dtype=np.int32)
    rng = np.random.default_rng(0)
    kc = rng.normal(0, 1, (NB, KVH, BS, D)).astype(np.float16)
    vc = rng.normal(0, 1, (NB, KVH, BS // 4, D, 4)).astype(np.float16)
    k = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    v = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    kc2, vc2 = oracle.cache_write(k, v, kc, vc, slots, BS, "f16")
    expect_k = kc.copy()
    expect_v = vc.copy()
    for i, (b, o) in enumerate([(2, 30), (1, 0), (6, 6)]):
        for h in range(KVH):
            for d in range(D):
                expect_k[b, h, o, d] = k[i, h, d]
                expect_v[b, h, o // 4, d, o % 4] = v[i, h, d]
    assert kc2.tobytes() == expect_k.tobytes()
    assert vc2.tobytes() == expect_v.tobytes()
    # inputs untouched
    assert not np.shares_memory(kc2, kc)


def test_negative_slot_is_skipped_and_duplicates_rejected():
    kc = np.zeros((2, 1, 4, 2), dtype=np.float16)
    vc = np.zeros((2, 1, 1, 2, 4), dtype=np.float16)
    k = np.ones((2, 1, 2), dtype=np.float16)
    kc2, vc2 = oracle.cache_write(k, k, kc, vc, np.array([-1, -1], dtype=np.int32), 4, "f16")
    assert not kc2.any() and not vc2.any()
    with pytest.raises(ValueError):
        oracle.cache_write(k, k, kc, vc, np.array([3, 3], dtype=np.int32), 4, "f16")
    with pytest.raises(ValueError):
        oracle.cache_write(k, k, kc, vc, np.array([8, 0], dtype=np.int32), 4, "f16")


def test_bf16_write_keeps_bits():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, (3, 2, 8), dtype=np.uint16)
    kc = np.zeros((4, 2, 4, 8), dtype=np.uint16)
    vc = np.zeros((4, 2, 1, 8, 4), dtype=np.uint16)
    kc2, vc2 = oracle.cache_write(bits, bits, kc, vc, np.array([0, 5, 15], dtype=np.int32), 4, "bf16")
    assert np.array_equal(kc2[1, :, 1, :], bits[1]) and np.array_equal(vc2[3, :, 0, :, 3], bits[2])


def test_fp8_write_codes():
    """e4m3fn(clamp(fp32(x) * fp32(1/scale))) against torch's cast of the same
    binary32 products (in range), and saturation beyond 448 * scale."""
    rng = np.random.default_rng(2)
    KVH, D, BS = 2, 16, 16
    x = rng.normal(0, 1, (4, KVH, D)).astype(np.float32)
    x[0, 0, 0] = 1e4                                        # saturates
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    kscale = float(np.float32(np.abs(x[1:]).max() / 448.0))
    kc = np.zeros((3, KVH, BS, D), dtype=np.uint8)
    vc = np.zeros((3, KVH, BS // 4, D, 4), dtype=np.uint8)
    slots = np.array([0, 17, 33, 47], dtype=np.int32)
    kc2, vc2 = oracle.cache_write(bits, bits, kc, vc, slots, BS, "e4m3fn", k_scale=kscale, v_scale=0.5)
    inv = np.float32(np.float32(1.0) / np.float32(kscale))
    prod = (xb.float().numpy() * inv).astype(np.float32)
    ref = torch.from_numpy(np.clip(prod, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, s in enumerate(slots):
        b, o = divmod(int(s), BS)
        assert np.array_equal(kc2[b, :, o, :], ref[i])
    assert kc2[0, 0, 0, 0] == 0x7E
    vref = torch.from_numpy(np.clip(xb.float().numpy() * np.float32(2.0), -448, 448)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(vc2[2, :, 3, :, 3], vref[3])


def test_write_then_decode_attends_the_new_token():
    """After the step's write, decoding with context_len + 1 equals decoding a
    pool where the token was placed by hand; with context_len it is unchanged."""
    ex = _example()
    page = ex["stated_by_the_page"]
    BS, KVH, D = page["block_size"], 2, 8
    table = np.array(page["block_table"], dtype=np.int32)
    L = np.array(page["cache_seqlens"], dtype=np.int32)
    rng = np.random.default_rng(3)
    kc = rng.normal(0, 1, (8, KVH, BS, D)).astype(np.float16)
    vc = rng.normal(0, 1, (8, KVH, BS // 4, D, 4)).astype(np.float16)
    q = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    k = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    v = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    slots = np.array(ex["derived_by_definition"]["new_token_slot"], dtype=np.int32)
    kc2, vc2 = oracle.cache_write(k, v, kc, vc, slots, BS, "f16")
    before = oracle.paged_decode(q, kc, vc, table, L, 0.3, KVH, BS, "f16", "f16")
    same = oracle.paged_decode(q, kc2, vc2, table, L, 0.3, KVH, BS, "f16", "f16")
    assert np.array_equal(before, same)
    after = oracle.paged_decode(q, kc2, vc2, table, L + 1, 0.3, KVH, BS, "f16", "f16")
    for s in range(3):
        for h in range(KVH):
            K = np.array([kc[table[s, t // BS], h, t % BS] for t in range(L[s])] + [k[s, h]], dtype=np.float64)
            V = np.array([vc[table[s, t // BS], h, (t % BS) // 4, :, t % 4] for t in range(L[s])] + [v[s, h]],
                         dtype=np.float64)
            x = float(np.float32(0.3)) * (K @ q[s, h].astype(np.float64))
            w = np.exp(x - x.max())
            np.testing.assert_allclose(after[s, h], (w / w.sum()) @ V, rtol=1e-12, atol=1e-14)
