"""Pins of the oracle's paged decode attention (CPU only).

Each check is independent of the oracle's own code path:
  * brute force: scalar Python loops that read every slot through the block
    table directly (no gather, no matmul), math.exp;
  * library special case: torch's scaled_dot_product_attention in float64 on
    the contiguous K/V the test itself scattered into the paged pool;
  * closed forms (one token, constant V, two tokens, q = 0, a needle);
  * invariances (relabelled physical ids, another block size, partitions).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _scatter(Kc, Vc, block_size, rng, spare=2):
    """Lay contiguous per-sequence K/V ([L_s, KVH, D] fp16 each) into a paged
    pool with randomly permuted physical blocks.  Returns the caches, table,
    lens.  Unused slots are left NaN (they must never be read)."""
    S = len(Kc)
    KVH, D = Kc[0].shape[1], Kc[0].shape[2]
    lens = [k.shape[0] for k in Kc]
    need = [-(-L // block_size) for L in lens]
    NB = sum(need) + spare
    perm = rng.permutation(NB)
    MB = max(max(need), 1) + 1
    table = -np.ones((S, MB), dtype=np.int32)
    kc = np.full((NB, KVH, block_size, D), np.nan, dtype=np.float16)
    vc = np.full((NB, KVH, block_size // 4, D, 4), np.nan, dtype=np.float16)
    nxt = 0
    for s in range(S):
        for j in range(need[s]):
            table[s, j] = perm[nxt]
            nxt += 1
        for t in range(lens[s]):
            b = table[s, t // block_size]
            o = t % block_size
            for h in range(KVH):
                for d in range(D):
                    kc[b, h, o, d] = Kc[s][t, h, d]
                    vc[b, h, o // 4, d, o % 4] = Vc[s][t, h, d]
    return kc, vc, table, np.array(lens, dtype=np.int32)


def _problem(rng, S=3, H=4, KVH=2, D=8, lens=(1, 17, 40), block_size=8, dist=1.0):
    Kc = [rng.normal(0, dist, (L, KVH, D)).astype(np.float16) for L in lens]
    Vc = [rng.normal(0, 1, (L, KVH, D)).astype(np.float16) for L in lens]
    q = rng.normal(0, 1, (S, H, D)).astype(np.float16)
    kc, vc, table, L = _scatter(Kc, Vc, block_size, rng)
    return q, Kc, Vc, kc, vc, table, L


def _brute(q, kc, vc, table, lens, scale, KVH, BS):
    """Scalar loops over slots read through the table."""
    S, H, D = q.shape
    G = H // KVH
    out = np.zeros((S, H, D))
    for s in range(S):
        for h in range(H):
            kvh = h // G
            xs = []
            for t in range(int(lens[s])):
                b = int(table[s][t // BS])
                o = t % BS
                acc = 0.0
                for d in range(D):
                    acc += float(q[s, h, d]) * float(kc[b, kvh, o, d])
                xs.append(float(np.float32(scale)) * acc)
            if not xs:
                continue
            m = max(xs)
            w = [math.exp(x - m) for x in xs]
            tot = math.fsum(w)
            for d in range(D):
                acc = 0.0
                for t in range(int(lens[s])):
                    b = int(table[s][t // BS])
                    o = t % BS
                    acc += w[t] * float(vc[b, kvh, o // 4, d, o % 4])
                out[s, h, d] = acc / tot
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, lens=(1, 17, 40), block_size=8)
    scale = 1 / math.sqrt(8)
    got = oracle.paged_decode(q, kc, vc, table, L, scale, 2, 8, "f16", "f16")
    ref = _brute(q, kc, vc, table, L, scale, 2, 8)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_brute_force_mha_and_empty_context():
    rng = np.random.default_rng(7)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=3, H=3, KVH=3, D=4, lens=(0, 5, 33), block_size=4)
    got = oracle.paged_decode(q, kc, vc, table, L, 0.5, 3, 4, "f16", "f16")
    ref = _brute(q, kc, vc, table, L, 0.5, 3, 4)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("H,KVH", [(4, 4), (8, 2), (6, 1)])
def test_sdpa_library_case(H, KVH):
    """torch scaled_dot_product_attention (float64, CPU) over the contiguous
    K/V, with kv head h // (H/KVH) expanded by repeat_interleave."""
    rng = np.random.default_rng(H * 10 + KVH)
    D, BS = 16, 16
    lens = (1, 16, 17, 100)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=4, H=H, KVH=KVH, D=D, lens=lens, block_size=BS)
    scale = float(np.float32(1 / math.sqrt(D)))
    got = oracle.paged_decode(q, kc, vc, table, L, scale, KVH, BS, "f16", "f16")
    for s in range(4):
        K = torch.from_numpy(Kc[s].astype(np.float64)).permute(1, 0, 2)   # [KVH, L, D]
        V = torch.from_numpy(Vc[s].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(H // KVH, dim=0)
        V = V.repeat_interleave(H // KVH, dim=0)
        Q = torch.from_numpy(q[s].astype(np.float64))[:, None, :]          # [H, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0]
        np.testing.assert_allclose(got[s], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_bf16_and_fp8_inputs_match_sdpa_on_dequantised_values():
    rng = np.random.default_rng(11)
    S, H, KVH, D, BS = 2, 4, 2, 16, 16
    lens = (20, 33)
    q = rng.normal(0, 1, (S, H, D)).astype(np.float32)
    qbits = (q.view(np.uint32) >> 16).astype(np.uint16)               # truncated to bf16
    qv = oracle.bf16_to_f64(qbits)
    codes_k = rng.integers(0, 256, (8, KVH, BS, D), dtype=np.uint8)
    codes_v = rng.integers(0, 256, (8, KVH, BS // 4, D, 4), dtype=np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x01                           # no NaN codes
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x02
    table = np.array([[3, 1, -1], [0, 6, 2]], dtype=np.int32)
    L = np.array(lens, dtype=np.int32)
    ks, vs = 0.03125, 0.0078125
    got = oracle.paged_decode(qbits, codes_k, codes_v, table, L, 0.25, KVH, BS, "bf16",
                              "e4m3fn", k_scale=ks, v_scale=vs)
    tk = torch.from_numpy(codes_k).view(torch.float8_e4m3fn).to(torch.float64) * ks
    tv = torch.from_numpy(codes_v).view(torch.float8_e4m3fn).to(torch.float64) * vs
    for s in range(S):
        rows = [(int(table[s, t // BS]), t % BS) for t in range(lens[s])]
        K = torch.stack([tk[b, :, o, :] for b, o in rows], 1)            # [KVH, L, D]
        V = torch.stack([tv[b, :, o // 4, :, o % 4] for b, o in rows], 1)
        K = K.repeat_interleave(H // KVH, 0)
        V = V.repeat_interleave(H // KVH, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qv[s])[:, None, :], K, V, scale=0.25)[:, 0]
        np.testing.assert_allclose(got[s], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_one_token_context_returns_v0():
    rng = np.random.default_rng(3)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=2, H=2, KVH=2, D=8, lens=(1, 1), block_size=4)
    got = oracle.paged_decode(q, kc, vc, table, L, 1.0, 2, 4, "f16", "f16")
    for s in range(2):
        assert np.array_equal(got[s], Vc[s][0].astype(np.float64))


def test_constant_v_and_weights_sum_to_one():
    rng = np.random.default_rng(4)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=2, H=2, KVH=1, D=8, lens=(9, 50), block_size=8)
    c = np.float16(-1.375)
    for s in range(2):
        Vc[s][:] = c
    kc2, vc2, table2, L2 = _scatter(Kc, Vc, 8, np.random.default_rng(0))
    got = oracle.paged_decode(q, kc2, vc2, table2, L2, 0.3, 1, 8, "f16", "f16")
    np.testing.assert_allclose(got, np.full(got.shape, float(c)), rtol=0, atol=1e-14)
    for s in range(2):
        _, probs = oracle.decode_sequence(q[s].astype(np.float64), kc2, vc2, table2[s], L2[s],
                                          0.3, 1, 8, "f16", return_probs=True)
        for p in probs:
            assert abs(math.fsum(p) - 1.0) < 1e-12
            assert np.all(p > 0)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(5)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=1, H=1, KVH=1, D=8, lens=(2,), block_size=4)
    scale = 0.7
    got = oracle.paged_decode(q, kc, vc, table, L, scale, 1, 4, "f16", "f16")[0, 0]
    x = [float(np.float32(scale)) * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], Kc[0][t, 0]))
         for t in range(2)]
    s0 = 1 / (1 + math.exp(x[1] - x[0]))
    s1 = 1 / (1 + math.exp(x[0] - x[1]))
    ref = s0 * Vc[0][0, 0].astype(np.float64) + s1 * Vc[0][1, 0].astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(6)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=2, H=2, KVH=2, D=8, lens=(5, 37), block_size=8)
    q[:] = 0
    got = oracle.paged_decode(q, kc, vc, table, L, 1.0, 2, 8, "f16", "f16")
    for s in range(2):
        ref = Vc[s].astype(np.float64).mean(axis=0)                    # [KVH, D]
        np.testing.assert_allclose(got[s], ref, rtol=1e-13, atol=1e-14)


def test_needle_selects_one_value():
    rng = np.random.default_rng(8)
    S, H, D, BS = 2, 2, 8, 8
    lens = (30, 45)
    q = rng.normal(0, 1, (S, H, D)).astype(np.float16)
    Kc = [rng.normal(0, 1, (L, H, D)).astype(np.float16) for L in lens]
    Vc = [rng.normal(0, 1, (L, H, D)).astype(np.float16) for L in lens]
    needles = [11, 44]
    for s, t in enumerate(needles):
        Kc[s][t] = (q[s] * 64).astype(np.float16)                     # x_t* dominates by > 100
    kc, vc, table, L = _scatter(Kc, Vc, BS, rng)
    got = oracle.paged_decode(q, kc, vc, table, L, 1.0, H, BS, "f16", "f16")
    for s, t in enumerate(needles):
        np.testing.assert_allclose(got[s], Vc[s][t].astype(np.float64), rtol=0, atol=1e-30)


def test_relabelled_physical_blocks_bit_identical():
    rng = np.random.default_rng(9)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=3, H=4, KVH=2, D=8, lens=(3, 26, 41), block_size=8)
    base = oracle.paged_decode(q, kc, vc, table, L, 0.4, 2, 8, "f16", "f16")
    NB = kc.shape[0]
    sigma = rng.permutation(NB)                # new id of old block b is sigma[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[sigma] = kc
    vc2[sigma] = vc
    t2 = np.where(table >= 0, sigma[np.maximum(table, 0)], -1).astype(np.int32)
    again = oracle.paged_decode(q, kc2, vc2, t2, L, 0.4, 2, 8, "f16", "f16")
    assert np.array_equal(base, again)


def test_block_size_invariance():
    rng = np.random.default_rng(10)
    lens = (7, 33, 64, 65)
    Kc = [rng.normal(0, 1, (L, 2, 16)).astype(np.float16) for L in lens]
    Vc = [rng.normal(0, 1, (L, 2, 16)).astype(np.float16) for L in lens]
    q = rng.normal(0, 1, (4, 2, 16)).astype(np.float16)
    outs = []
    for bs in (4, 16, 32):
        kc, vc, table, L = _scatter(Kc, Vc, bs, np.random.default_rng(bs))
        outs.append(oracle.paged_decode(q, kc, vc, table, L, 0.25, 2, bs, "f16", "f16"))
    # same logical K/V, only the tiling differs: equal up to summation order
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(outs[1], outs[2], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("P", [8, 16, 48, 512])
def test_partition_merge_equals_unpartitioned(P):
    rng = np.random.default_rng(12)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=4, H=4, KVH=2, D=8, lens=(0, 8, 9, 100), block_size=8)
    ref = oracle.paged_decode(q, kc, vc, table, L, 0.5, 2, 8, "f16", "f16")
    got, parts = oracle.paged_decode_partitioned(q, kc, vc, table, L, 0.5, 2, 8, "f16", "f16", P)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    for (s, h), pp in parts.items():
        assert len(pp) == oracle.num_logical_blocks(int(L[s]), P)
        for m, l, o in pp:
            assert l >= 1.0                      # the max term contributes e^0
            assert np.all(np.isfinite(o))


def test_one_partition_merge_is_exact():
    rng = np.random.default_rng(13)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=2, H=2, KVH=2, D=8, lens=(5, 31), block_size=8)
    _, parts = oracle.paged_decode_partitioned(q, kc, vc, table, L, 0.5, 2, 8, "f16", "f16", 32)
    for pp in parts.values():
        assert len(pp) == 1
        assert np.array_equal(oracle.merge_partials(pp), pp[0][2])


def test_partition_triples_against_brute_force():
    """Each partition's (m, l, o) against scalar loops over its tokens."""
    rng = np.random.default_rng(14)
    q, Kc, Vc, kc, vc, table, L = _problem(rng, S=1, H=1, KVH=1, D=4, lens=(21,), block_size=4)
    _, parts = oracle.paged_decode_partitioned(q, kc, vc, table, L, 0.9, 1, 4, "f16", "f16", 8)
    pp = parts[(0, 0)]
    for p, (m, l, o) in enumerate(pp):
        ts = range(8 * p, min(8 * p + 8, 21))
        xs = [float(np.float32(0.9)) * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], Kc[0][t, 0]))
              for t in ts]
        mm = max(xs)
        w = [math.exp(x - mm) for x in xs]
        assert m == pytest.approx(mm, rel=1e-14)
        assert l == pytest.approx(math.fsum(w), rel=1e-13)
        ref = [math.fsum(wi * float(Vc[0][t, 0, d]) for wi, t in zip(w, ts)) / math.fsum(w) for d in range(4)]
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
