"""Pins of the oracle's varlen / chunked prefill over the paged cache (CPU)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    with open(os.path.join(GOLDEN, "varlen_cu_seqlens_example.json")) as f:
        return json.load(f)["stated_by_the_page"]


def _paged(rng, lens, KVH, BS, D, extra=3, dt=np.float16):
    """Random pool and block tables (permuted blocks) holding len tokens per
    sequence, plus the same K/V as contiguous per-sequence arrays."""
    need = [-(-L // BS) for L in lens]
    NB = sum(need) + extra
    perm = rng.permutation(NB)
    MB = max(max(need), 1)
    table = np.full((len(lens), MB), -1, dtype=np.int32)
    k = rng.normal(0, 1, (NB, KVH, BS, D)).astype(dt)
    v = rng.normal(0, 1, (NB, KVH, BS // 4, D, 4)).astype(dt)
    used = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[used:used + n]
        used += n
    return k, v, table


def _rows(k, v, table, s, L, kvh, BS):
    K = np.array([k[table[s, t // BS], kvh, t % BS] for t in range(L)], dtype=np.float64)
    V = np.array([v[table[s, t // BS], kvh, (t % BS) // 4, :, t % 4] for t in range(L)],
                 dtype=np.float64)
    return K.reshape(L, -1), V.reshape(L, -1)


def test_cu_seqlens_example():
    """The wiki's varlen example: which request each packed Q and K token
    belongs to, and the maximum lengths."""
    ex = _example()
    cq, ck = ex["cu_seq_lens_q"], ex["cu_seq_lens_k"]
    assert list(np.cumsum([0] + ex["query_lens"])) == cq
    assert list(np.cumsum([0] + ex["key_lens"])) == ck
    assert oracle.request_index(cq) == ex["q_request_index"]
    assert oracle.request_index(ck) == ex["k_request_index"]
    assert len(oracle.request_index(cq)) == ex["q_packed_tokens"]
    assert len(oracle.request_index(ck)) == ex["k_packed_tokens"]
    assert max(ex["query_lens"]) == ex["max_seqlen_q"] and max(ex["key_lens"]) == ex["max_seqlen_k"]
    with pytest.raises(ValueError):
        oracle.request_index([0, 3, 2])


def test_example_shapes_with_causal_alignment():
    """The example's lengths as a chunked-prefill batch (queries are each
    sequence's last positions): r0 has no keys (zeros); r1's three queries
    sit before, before and at its one key (zeros, zeros, that key's V); r2's
    single query attends all 7 keys (the decode definition)."""
    ex = _example()
    rng = np.random.default_rng(0)
    KVH, H, D, BS = 2, 4, 8, 4
    lens = ex["key_lens"]
    k, v, table = _paged(rng, lens, KVH, BS, D)
    q = rng.normal(0, 1, (ex["q_packed_tokens"], H, D)).astype(np.float16)
    cu = np.array(ex["cu_seq_lens_q"], dtype=np.int32)
    L = np.array(lens, dtype=np.int32)
    out = oracle.paged_prefill(q, k, v, table, cu, L, 0.35, KVH, BS, "f16", "f16")
    assert not out[0:10].any() and not out[10:12].any()
    for h in range(H):
        b = table[1, 0]
        assert np.array_equal(out[12, h], v[b, h // 2, 0, :, 0].astype(np.float64))
    dec = oracle.paged_decode(q[13:14], k, v, table[2:3], L[2:3], 0.35, KVH, BS, "f16", "f16")
    np.testing.assert_allclose(out[13], dec[0], rtol=1e-12, atol=1e-14)


def test_single_query_per_sequence_is_decode():
    rng = np.random.default_rng(1)
    KVH, H, D, BS = 2, 6, 16, 16
    lens = [1, 15, 16, 17, 70]
    k, v, table = _paged(rng, lens, KVH, BS, D)
    q = rng.normal(0, 1, (5, H, D)).astype(np.float16)
    cu = np.arange(6, dtype=np.int32)
    L = np.array(lens, dtype=np.int32)
    out = oracle.paged_prefill(q, k, v, table, cu, L, 0.2, KVH, BS, "f16", "f16")
    dec = oracle.paged_decode(q, k, v, table, L, 0.2, KVH, BS, "f16", "f16")
    np.testing.assert_allclose(out, dec, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_sdpa_with_explicit_mask(causal):
    """torch scaled_dot_product_attention in float64 on the gathered K/V, with
    a boolean mask allowing key j for query i iff j <= K - n + i (causal)."""
    rng = np.random.default_rng(2)
    KVH, H, D, BS = 2, 4, 16, 16
    lens = [9, 40, 33]
    qlens = [9, 5, 12]
    k, v, table = _paged(rng, lens, KVH, BS, D)
    cu = np.cumsum([0] + qlens).astype(np.int32)
    q = rng.normal(0, 1, (cu[-1], H, D)).astype(np.float16)
    out = oracle.paged_prefill(q, k, v, table, cu, np.array(lens, dtype=np.int32), 0.25, KVH, BS,
                               "f16", "f16", causal=causal)
    for s, (Ks, n) in enumerate(zip(lens, qlens)):
        for kvh in range(KVH):
            K, V = _rows(k, v, table, s, Ks, kvh, BS)
            allow = np.ones((n, Ks), dtype=bool)
            if causal:
                allow = np.arange(Ks)[None, :] <= (Ks - n + np.arange(n))[:, None]
            for h in (2 * kvh, 2 * kvh + 1):
                qq = torch.from_numpy(q[cu[s]:cu[s + 1], h].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
                    attn_mask=torch.from_numpy(allow)[None, None],
                    scale=float(np.float32(0.25)))[0, 0].numpy()
                np.testing.assert_allclose(out[cu[s]:cu[s + 1], h], ref, rtol=1e-10, atol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    KVH, H, D, BS = 1, 2, 4, 4
    lens, qlens = [6, 3], [4, 3]
    k, v, table = _paged(rng, lens, KVH, BS, D)
    cu = np.cumsum([0] + qlens).astype(np.int32)
    q = rng.normal(0, 1, (cu[-1], H, D)).astype(np.float16)
    out = oracle.paged_prefill(q, k, v, table, cu, np.array(lens, dtype=np.int32), 0.5, KVH, BS,
                               "f16", "f16")
    sc = float(np.float32(0.5))
    for s in range(2):
        for i in range(qlens[s]):
            for h in range(H):
                last = lens[s] - qlens[s] + i
                xs, vs = [], []
                for t in range(last + 1):
                    b, o = table[s, t // BS], t % BS
                    xs.append(sc * sum(float(q[cu[s] + i, h, d]) * float(k[b, 0, o, d])
                                       for d in range(D)))
                    vs.append([float(v[b, 0, o // 4, d, o % 4]) for d in range(D)])
                mx = max(xs)
                w = [np.exp(x - mx) for x in xs]
                ref = [sum(w[t] * vs[t][d] for t in range(len(w))) / sum(w) for d in range(D)]
                np.testing.assert_allclose(out[cu[s] + i, h], ref, rtol=1e-12, atol=1e-14)


def test_two_chunks_equal_one():
    """A prompt prefilled in one chunk equals the same prompt in two chunks
    (the second chunk's queries see the first chunk's keys): the positions
    of the queries are the last n of the K cached ones."""
    rng = np.random.default_rng(4)
    KVH, H, D, BS = 2, 4, 8, 16
    Ktot, a = 37, 20
    k, v, table = _paged(rng, [Ktot], KVH, BS, D)
    q = rng.normal(0, 1, (Ktot, H, D)).astype(np.float16)
    one = oracle.paged_prefill(q, k, v, table, np.array([0, Ktot], dtype=np.int32),
                               np.array([Ktot], dtype=np.int32), 0.3, KVH, BS, "f16", "f16")
    first = oracle.paged_prefill(q[:a], k, v, table, np.array([0, a], dtype=np.int32),
                                 np.array([a], dtype=np.int32), 0.3, KVH, BS, "f16", "f16")
    second = oracle.paged_prefill(q[a:], k, v, table, np.array([0, Ktot - a], dtype=np.int32),
                                  np.array([Ktot], dtype=np.int32), 0.3, KVH, BS, "f16", "f16")
    np.testing.assert_allclose(np.concatenate([first, second]), one, rtol=1e-12, atol=1e-14)


def test_future_keys_do_not_matter():
    """Changing keys and values after query i's position leaves its output
    unchanged (causal); the non-causal output changes."""
    rng = np.random.default_rng(5)
    KVH, H, D, BS = 1, 1, 8, 16
    k, v, table = _paged(rng, [30], KVH, BS, D)
    q = rng.normal(0, 1, (10, H, D)).astype(np.float16)
    cu = np.array([0, 10], dtype=np.int32)
    L = np.array([30], dtype=np.int32)
    base = oracle.paged_prefill(q, k, v, table, cu, L, 0.3, KVH, BS, "f16", "f16")
    base_nc = oracle.paged_prefill(q, k, v, table, cu, L, 0.3, KVH, BS, "f16", "f16", causal=False)
    k2, v2 = k.copy(), v.copy()
    t = 29                                             # last position: only query 9 sees it
    b, o = table[0, t // BS], t % BS
    k2[b, 0, o] = np.float16(3.0)
    v2[b, 0, o // 4, :, o % 4] = np.float16(-5.0)
    pert = oracle.paged_prefill(q, k2, v2, table, cu, L, 0.3, KVH, BS, "f16", "f16")
    pert_nc = oracle.paged_prefill(q, k2, v2, table, cu, L, 0.3, KVH, BS, "f16", "f16",
                                   causal=False)
    assert np.array_equal(pert[:9], base[:9]) and not np.array_equal(pert[9], base[9])
    assert not np.array_equal(pert_nc[0], base_nc[0])
