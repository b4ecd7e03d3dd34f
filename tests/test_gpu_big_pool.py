"""Decode and block copies over a pool larger than 4 GiB, through the C ABI: a small workload's
blocks are moved to ids whose tiles start past 4 GiB of each cache (a pool of
5 GiB per cache, NaN everywhere else), so every tile address and every slot
the fused step stores needs more than 32 bits of byte offset.  The results
must be those the oracle gives on the original small pool: the output within
the tolerance, the stored token's bytes exact.  Both decode kernels (one query
head per kv head on the vector ALU, grouped heads on the matrix cores), 16-bit
and fp8 caches, in one pass with the append and split into partitions; and
block copies to and from ids past 4 GiB."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_78_amd as pa
import workloads
from gpu_helpers import as_f64, assert_close, oracle_arrays, oracle_decode, tol_of
from workloads import to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _workload(qd, cache, G):
    H, KVH, BS = 2 * G, 2, 16
    if cache == "e4m3fn":
        return workloads.poison_unused_slots(workloads.fp8_shared_prefix(
            seed=81, num_seqs=6, median=150.0, cap=400, num_heads=H, num_kv_heads=KVH,
            head_size=128, block_size=BS, prefix_tokens=2 * BS))
    return workloads.poison_unused_slots(workloads.gqa(
        seed=82, num_seqs=6, len_range=(1, 300), num_heads=H, num_kv_heads=KVH, head_size=128,
        block_size=BS, dtype=qd, lengths=[1, BS - 1, BS, 5 * BS + 3, 257, 300]))


def _relocate(wl):
    """(k pool, v pool, table, slots, moved ids, original ids) on the device."""
    BS = wl.block_size
    table = wl.block_table.clone()
    slots = wl.slot_mapping.clone()
    used = sorted({int(x) for x in table.flatten().tolist() if x >= 0} |
                  {int(x) // BS for x in slots.tolist() if x >= 0})
    block_bytes = wl.k_cache[0].numel() * wl.k_cache.element_size()
    nb_big = (5 << 30) // block_bytes
    first = ((4 << 30) + block_bytes - 1) // block_bytes
    new_ids = {old: first + 5 + 41 * i for i, old in enumerate(reversed(used))}
    assert max(new_ids.values()) < nb_big
    for s in range(table.shape[0]):
        for j in range(table.shape[1]):
            if table[s, j] >= 0:
                table[s, j] = new_ids[int(table[s, j])]
    for i, sl in enumerate(slots.tolist()):
        if sl >= 0:
            slots[i] = new_ids[sl // BS] * BS + sl % BS
    idx = torch.tensor([new_ids[o] for o in used], dtype=torch.int64, device=DEV)
    pools = []
    for c in (wl.k_cache, wl.v_cache):
        t = torch.empty((nb_big,) + tuple(c.shape[1:]), dtype=c.dtype, device=DEV)
        if wl.cache_dtype == "e4m3fn":
            t.view(torch.uint8).fill_(0x7F)
        else:
            t.fill_(float("nan"))
        t[idx] = c[torch.tensor(used, dtype=torch.int64)].to(DEV)
        pools.append(t)
    return pools[0], pools[1], table.to(DEV), slots.to(DEV), idx, used


@pytest.mark.parametrize("mode", ["append", "partitioned"])
@pytest.mark.parametrize("qd,cache,G", [("f16", "f16", 1), ("bf16", "bf16", 4),
                                        ("bf16", "e4m3fn", 8), ("f16", "e4m3fn", 1)])
def test_decode_blocks_past_4gib(qd, cache, G, mode):
    wl = _workload(qd, cache, G)
    if qd == "f16" and cache == "e4m3fn":
        # the bf16 queries and new tokens (N(0,1)) are exact in f16
        wl = workloads.synth.replace(wl, q=wl.q.to(torch.float16), new_k=wl.new_k.to(torch.float16),
                                     new_v=wl.new_v.to(torch.float16), q_dtype="f16")
    what = f"pool past 4 GiB {qd}/{cache} G{G} {mode}"
    print(f"[big pool] {what}", flush=True)
    kp, vp, table, slots, idx, used = _relocate(wl)
    g = wl.to(DEV)
    atol, rtol = tol_of(wl)
    if mode == "append":
        out = pa.decode_append(g.q, g.new_k, g.new_v, kp, vp, slots, table, g.context_lens,
                               wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale)
        torch.cuda.synchronize()
        a = oracle_arrays(wl)
        ref, kc, vc = oracle.decode_append(a["q"], to_numpy_bits(wl.new_k),
                                           to_numpy_bits(wl.new_v), a["k"], a["v"],
                                           wl.slot_mapping.cpu().numpy(), a["table"], a["lens"],
                                           wl.scale, wl.num_kv_heads, wl.block_size, wl.q_dtype,
                                           wl.cache_dtype, wl.k_scale, wl.v_scale)
        assert_close(as_f64(out), ref, atol, rtol, what)
        for t, want in ((kp, kc), (vp, vc)):
            got = to_numpy_bits(t[idx].cpu())
            assert got.tobytes() == np.ascontiguousarray(want[used]).tobytes(), what
    else:
        maxL = int(wl.context_lens.max())
        out = pa.decode_partitioned(g.q, kp, vp, table, g.context_lens, wl.scale,
                                    2 * wl.block_size, maxL, wl.k_scale, wl.v_scale)
        torch.cuda.synchronize()
        assert_close(as_f64(out), oracle_decode(wl), atol, rtol, what)
    del kp, vp
    torch.cuda.empty_cache()


def test_copy_blocks_past_4gib():
    """Block copies between ids below and past 4 GiB of a 5 GiB pool (each way,
    and both past it): the destination blocks must hold what the oracle's copy
    gives on the same blocks gathered into a small pool."""
    print("[big pool] copy_blocks", flush=True)
    KVH, BS, D = 2, 16, 128
    block_bytes = KVH * BS * D * 2
    nb = (5 << 30) // block_bytes
    hi = (4 << 30) // block_bytes + 7
    pairs = [(hi + 3, 11), (12, hi + 100), (hi + 250, hi + 999), (nb - 1, 13), (14, nb - 2)]
    ids = sorted({i for pr in pairs for i in pr})
    gen = torch.Generator().manual_seed(83)
    small_k = torch.randn((len(ids), KVH, BS, D), generator=gen).to(torch.float16)
    small_v = torch.randn((len(ids), KVH, BS // 4, D, 4), generator=gen).to(torch.float16)
    k = torch.full((nb, KVH, BS, D), float("nan"), dtype=torch.float16, device=DEV)
    v = torch.full((nb, KVH, BS // 4, D, 4), float("nan"), dtype=torch.float16, device=DEV)
    idx = torch.tensor(ids, dtype=torch.int64, device=DEV)
    k[idx] = small_k.to(DEV)
    v[idx] = small_v.to(DEV)
    mapping = torch.tensor(pairs, dtype=torch.int32, device=DEV)
    pa.copy_blocks(k, v, k, v, mapping)
    torch.cuda.synchronize()
    pos = {b: i for i, b in enumerate(ids)}
    small_map = np.array([[pos[a], pos[b]] for a, b in pairs], dtype=np.int32)
    sk, sv = to_numpy_bits(small_k), to_numpy_bits(small_v)
    want_k, want_v = oracle.copy_blocks(sk, sv, sk, sv, small_map)
    assert to_numpy_bits(k[idx].cpu()).tobytes() == np.ascontiguousarray(want_k).tobytes()
    assert to_numpy_bits(v[idx].cpu()).tobytes() == np.ascontiguousarray(want_v).tobytes()
    del k, v
    torch.cuda.empty_cache()
