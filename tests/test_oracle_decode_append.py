"""Pins of the oracle's one-call decode step (cache write + attention over the
context and the new token), CPU only."""
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


def _pool(rng, NB, KVH, BS, D, dt=np.float16):
    kc = rng.normal(0, 1, (NB, KVH, BS, D)).astype(dt)
    vc = rng.normal(0, 1, (NB, KVH, BS // 4, D, 4)).astype(dt)
    return kc, vc


def test_worked_example_by_hand():
    """'Paged attention' wiki decode example (block size 32, tables
    [[2], [0, 1], [3, 5, 6]], cached lengths 30, 32, 70): each query attends
    over its cached tokens, gathered one by one by the position rule, and its
    new token; the new token lands in slots 94, 32, 198."""
    ex = _example()
    page = ex["stated_by_the_page"]
    BS, KVH, H, D = page["block_size"], 2, 4, 8
    table = np.array(page["block_table"], dtype=np.int32)
    L = np.array(page["cache_seqlens"], dtype=np.int32)
    slots = np.array(ex["derived_by_definition"]["new_token_slot"], dtype=np.int32)
    rng = np.random.default_rng(11)
    kc, vc = _pool(rng, 8, KVH, BS, D)
    q = rng.normal(0, 1, (3, H, D)).astype(np.float16)
    k = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    v = rng.normal(0, 1, (3, KVH, D)).astype(np.float16)
    out, kc2, vc2 = oracle.decode_append(q, k, v, kc, vc, slots, table, L, 0.25, KVH, BS,
                                         "f16", "f16")
    for s in range(3):
        for h in range(H):
            g = h // (H // KVH)
            rows_k = [kc[table[s, t // BS], g, t % BS] for t in range(L[s])] + [k[s, g]]
            rows_v = [vc[table[s, t // BS], g, (t % BS) // 4, :, t % 4] for t in range(L[s])]
            rows_v.append(v[s, g])
            K = np.array(rows_k, dtype=np.float64)
            V = np.array(rows_v, dtype=np.float64)
            x = float(np.float32(0.25)) * (K @ q[s, h].astype(np.float64))
            w = np.exp(x - x.max())
            np.testing.assert_allclose(out[s, h], (w / w.sum()) @ V, rtol=1e-12, atol=1e-14)
    # the caches are exactly the cache write's, new tokens at the page's slots
    for i, (b, o) in enumerate([(2, 30), (1, 0), (6, 6)]):
        assert np.array_equal(kc2[b, :, o], k[i])
        assert np.array_equal(vc2[b, :, o // 4, :, o % 4], v[i])


@pytest.mark.parametrize("cache_fmt", ["bf16", "e4m3fn"])
def test_equals_write_then_decode_one_longer(cache_fmt):
    """With each new token at position L's slot, one decode step equals the
    write followed by a decode over L + 1 tokens (fp8: the new token enters
    with its quantised value, read back through the cache)."""
    rng = np.random.default_rng(12)
    S, KVH, H, D, BS, NB, MB = 5, 2, 8, 16, 16, 40, 6
    L = np.array([0, 1, 15, 16, 70], dtype=np.int32)
    table = np.full((S, MB), -1, dtype=np.int32)
    perm = rng.permutation(NB)
    used = 0
    for s in range(S):
        n = (int(L[s]) + 1 + BS - 1) // BS
        table[s, :n] = perm[used:used + n]
        used += n
    slots = np.array([oracle.next_slot(table[s], L[s], BS) for s in range(S)], dtype=np.int32)
    xb = torch.randn(NB, KVH, BS, D, dtype=torch.float32) * 3
    xv = torch.randn(NB, KVH, BS // 4, D, 4, dtype=torch.float32) * 3
    if cache_fmt == "bf16":
        kc = xb.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        vc = xv.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ks = vs = 1.0
    else:
        kc = xb.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        vc = xv.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ks, vs = 0.02, 0.035
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bf(rng.normal(0, 1, (S, H, D)).astype(np.float32))
    k = bf(rng.normal(0, 2, (S, KVH, D)).astype(np.float32))
    v = bf(rng.normal(0, 2, (S, KVH, D)).astype(np.float32))
    out, kc2, vc2 = oracle.decode_append(q, k, v, kc, vc, slots, table, L, 0.2, KVH, BS, "bf16",
                                         cache_fmt, ks, vs)
    kw, vw = oracle.cache_write(k, v, kc, vc, slots, BS, cache_fmt, ks, vs)
    assert kc2.tobytes() == kw.tobytes() and vc2.tobytes() == vw.tobytes()
    ref = oracle.paged_decode(q, kw, vw, table, L + 1, 0.2, KVH, BS, "bf16", cache_fmt, ks, vs)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_empty_context_gives_the_new_value():
    """One token: its softmax weight is 1, so every head of a kv group returns
    the new V row as stored (fp8: torch's e4m3fn cast of x / scale, times
    scale)."""
    rng = np.random.default_rng(13)
    KVH, H, D, BS = 2, 6, 32, 16
    kc = np.zeros((3, KVH, BS, D), dtype=np.uint8)
    vc = np.zeros((3, KVH, BS // 4, D, 4), dtype=np.uint8)
    x = rng.normal(0, 4, (1, KVH, D)).astype(np.float32)
    vb = torch.from_numpy(x).to(torch.float16)
    v = vb.numpy()
    k = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    q = rng.normal(0, 1, (1, H, D)).astype(np.float16)
    table = np.array([[1, -1]], dtype=np.int32)
    out, _, _ = oracle.decode_append(q, k, v, kc, vc, np.array([16], dtype=np.int32), table,
                                     np.array([0], dtype=np.int32), 0.1, KVH, BS, "f16", "e4m3fn",
                                     0.5, 0.125)
    inv = np.float32(1.0) / np.float32(0.125)
    stored = torch.from_numpy(np.clip(vb.float().numpy() * inv, -448, 448)).to(
        torch.float8_e4m3fn).float().numpy().astype(np.float64) * 0.125
    for h in range(H):
        np.testing.assert_array_equal(out[0, h], stored[0, h // 3])


def test_slot_does_not_change_the_attention():
    """The new token is taken from the inputs: where it is stored (another
    block, or nowhere) does not change the result; only the caches differ."""
    rng = np.random.default_rng(14)
    KVH, H, D, BS = 1, 2, 8, 16
    kc, vc = _pool(rng, 4, KVH, BS, D)
    q = rng.normal(0, 1, (1, H, D)).astype(np.float16)
    k = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    v = rng.normal(0, 1, (1, KVH, D)).astype(np.float16)
    table = np.array([[2, 0]], dtype=np.int32)
    L = np.array([20], dtype=np.int32)
    outs = []
    for slot in (4, 63, -1):
        out, kc2, _ = oracle.decode_append(q, k, v, kc, vc, np.array([slot], dtype=np.int32),
                                           table, L, 0.5, KVH, BS, "f16", "f16")
        outs.append(out)
        if slot < 0:
            assert kc2.tobytes() == kc.tobytes()
        else:
            assert np.array_equal(kc2[slot // BS, 0, slot % BS], k[0, 0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
