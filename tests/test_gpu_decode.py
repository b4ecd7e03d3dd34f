"""GPU parity of pa_decode / pa_decode_partitioned / pa_reduce / pa_cache_write
against the CPU oracle, through the C ABI (python binding)."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_78_amd as pa
import workloads
from gpu_helpers import as_f64, assert_close, bits16, oracle_arrays, oracle_decode, tol_of
from workloads import to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(wl):
    return wl.to(DEV)


def _decode(wl, lens=None, out=None):
    L = wl.context_lens if lens is None else lens
    return pa.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, L, wl.scale,
                     k_scale=wl.k_scale, v_scale=wl.v_scale, out=out)


# ----------------------------------------------------------------------------
# the pages' worked example: decode, cache write, decode again

def test_worked_example_decode_write_decode():
    wl = workloads.poison_unused_slots(workloads.worked_example())
    g = _gpu(wl)
    out = _decode(g)
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    assert_close(as_f64(out), oracle_decode(wl), atol, rtol, "decode over [30, 32, 70]")

    pa.cache_write(g.new_k, g.new_v, g.k_cache, g.v_cache, g.slot_mapping)
    torch.cuda.synchronize()
    a = oracle_arrays(wl)
    kc, vc = oracle.cache_write(to_numpy_bits(wl.new_k), to_numpy_bits(wl.new_v), a["k"], a["v"],
                                wl.slot_mapping.numpy(), wl.block_size, "f16")
    assert to_numpy_bits(g.k_cache).tobytes() == kc.tobytes()
    assert to_numpy_bits(g.v_cache).tobytes() == vc.tobytes()

    lens1 = g.context_lens + 1
    out1 = _decode(g, lens1)
    torch.cuda.synchronize()
    ref1 = oracle.paged_decode(a["q"], kc, vc, a["table"], a["lens"] + 1, wl.scale,
                               wl.num_kv_heads, wl.block_size, "f16", "f16")
    assert_close(as_f64(out1), ref1, atol, rtol, "decode over [31, 33, 71]")


# ----------------------------------------------------------------------------
# small MHA workloads over every built head size / block size / dtype

def _small(dtype, D, BS, H=4, KVH=None, seed=5, lens=None):
    """7 sequences of up to 300 tokens; `lens` fixes the first lengths (edge
    cases: 0, 1, BS-1, BS, BS+1, several tiles, ragged tails).  Slots outside
    every context hold NaN."""
    if KVH is None:
        wl = workloads.llama7b_mha(seed=seed, num_seqs=7, len_range=(1, 300), num_heads=H,
                                   head_size=D, block_size=BS, dtype=dtype, lengths=lens)
    else:
        wl = workloads.gqa(seed=seed, num_seqs=7, len_range=(1, 300), num_heads=H,
                           num_kv_heads=KVH, head_size=D, block_size=BS, dtype=dtype,
                           lengths=lens)
    return workloads.poison_unused_slots(wl)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(128, 16), (128, 32), (64, 16), (64, 32)])
def test_mha_small_against_oracle(dtype, D, BS):
    wl = _small(dtype, D, BS, lens=[1, BS - 1, BS, BS + 1, 5 * BS + 3, 257])
    out = _decode(_gpu(wl))
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    assert_close(as_f64(out), oracle_decode(wl), atol, rtol, f"{dtype} D{D} BS{BS}")


@pytest.mark.parametrize("G", [2, 8])
def test_grouped_heads_small_against_oracle(G):
    wl = _small("bf16", 128, 16, H=2 * G, KVH=2, lens=[1, 15, 16, 17, 99])
    out = _decode(_gpu(wl))
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    assert_close(as_f64(out), oracle_decode(wl), atol, rtol, f"G={G}")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("G", [1, 8])
def test_negative_and_zero_scale(scale, G):
    """A negative scale (logits change sign) and a zero scale (uniform
    weights over the context), one head per kv head and grouped heads."""
    wl = _small("f16" if G == 1 else "bf16", 128, 16, H=2 * G, KVH=2, lens=[1, 15, 16, 17, 99])
    wl = workloads.synth.replace(wl, scale=scale)
    out = _decode(_gpu(wl))
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    assert_close(as_f64(out), oracle_decode(wl), atol, rtol, f"scale {scale} G={G}")


@pytest.mark.parametrize("S,G", [(300, 1), (300, 8), (1024, 1), (1025, 1), (1100, 1), (1100, 4)])
def test_many_sequences(S, G):
    """More sequences than one lane set caches for the longest-first ranking
    (256: lengths are read again in its second pass) and than the ranking
    covers at all (1024, the last count it orders; beyond: index order), one
    head per kv head and grouped;
    every row against the oracle (the output starts as NaN, so a sequence
    the ranking skipped cannot pass)."""
    if G == 1:
        wl = workloads.llama7b_mha(seed=51, num_seqs=S, len_range=(0, 120), num_heads=2,
                                   head_size=64, block_size=16)
    else:
        wl = workloads.gqa(seed=51, num_seqs=S, len_range=(0, 120), num_heads=2 * G,
                           num_kv_heads=2, head_size=64, block_size=16)
    wl = workloads.poison_unused_slots(wl, covered=(wl.context_lens + 1).tolist())
    print(f"[decode] {S} sequences, G={G}", flush=True)
    g = _gpu(wl)
    lens = (g.context_lens + 1).contiguous()
    out = _decode(g, lens=lens)
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    ref = oracle_decode(wl, lens=lens.cpu().numpy())
    assert_close(as_f64(out), ref, atol, rtol, f"S={S} G={G}, every row")


# ----------------------------------------------------------------------------
# identities that hold bit for bit

def test_one_token_context_returns_v0_exactly():
    wl = _small("f16", 128, 16)
    L = torch.ones(wl.num_seqs, dtype=torch.int32)
    wl = workloads.poison_unused_slots(workloads.synth.replace(wl, context_lens=L))
    g = _gpu(wl)
    out = _decode(g)
    torch.cuda.synchronize()
    vc = wl.v_cache
    for s in range(wl.num_seqs):
        b = int(wl.block_table[s, 0])
        v0 = vc[b, :, 0, :, 0]                              # [KVH, D]
        assert np.array_equal(bits16(out[s]), bits16(v0)), s


def test_constant_values_give_that_constant_exactly():
    wl = _small("bf16", 128, 16, lens=[3, 200, 33])
    c = -1.375
    v = torch.full_like(wl.v_cache, c)
    wl = workloads.poison_unused_slots(workloads.synth.replace(wl, v_cache=v))
    out = _decode(_gpu(wl))
    torch.cuda.synchronize()
    assert torch.all(out.float().cpu() == c)


def test_needle_selects_its_value_exactly():
    wl = _small("f16", 128, 16, lens=[40, 250, 17, 16, 1, 300, 129])
    k = wl.k_cache.clone()
    needles = [39, 3, 16, 0, 0, 299, 64]
    for s, t in enumerate(needles):
        b = int(wl.block_table[s, t // 16])
        # K[t*] = 16 q: its logit beats every other one by far more than 150
        k[b, :, t % 16, :] = (wl.q[s].float() * 16).to(torch.float16)
    wl = workloads.synth.replace(wl, k_cache=k)
    out = _decode(_gpu(wl))
    torch.cuda.synchronize()
    for s, t in enumerate(needles):
        b = int(wl.block_table[s, t // 16])
        o = t % 16
        assert np.array_equal(bits16(out[s]), bits16(wl.v_cache[b, :, o // 4, :, o % 4])), s


def test_relabelled_blocks_and_repeat_runs_are_bit_identical():
    wl = _small("f16", 128, 16)
    g = _gpu(wl)
    base = _decode(g).clone()
    again = _decode(g)
    torch.cuda.synchronize()
    assert torch.equal(base, again)
    sigma = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(0))
    k2 = torch.empty_like(wl.k_cache)
    v2 = torch.empty_like(wl.v_cache)
    k2[sigma] = wl.k_cache
    v2[sigma] = wl.v_cache
    t = wl.block_table.long()
    t2 = torch.where(t >= 0, sigma[t.clamp(min=0)], torch.full_like(t, -1)).to(torch.int32)
    wl2 = workloads.synth.replace(wl, k_cache=k2, v_cache=v2, block_table=t2)
    out2 = _decode(_gpu(wl2))
    torch.cuda.synchronize()
    assert torch.equal(base, out2)


def test_empty_context_gives_zeros_and_bad_entries_give_nan_rows():
    wl = _small("f16", 128, 16, lens=[0, 40, 50, 60, 1])
    t = wl.block_table.clone()
    t[1, 1] = -1                      # inside the 40-token context
    t[2, 0] = wl.num_blocks           # out of the pool
    L = wl.context_lens.clone()
    L[3] = wl.max_blocks_per_seq * 16 + 1      # longer than the table
    L[4] = -5
    wl = workloads.synth.replace(wl, block_table=t, context_lens=L)
    out = _decode(_gpu(wl)).float().cpu()
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    for s in (1, 2, 3, 4):
        assert torch.all(torch.isnan(out[s])), s
    good = oracle_decode(wl, seqs=[5, 6])
    atol, rtol = tol_of(wl)
    assert_close(out[5:7].double().numpy(), good, atol, rtol, "rows after the bad ones")


# ----------------------------------------------------------------------------
# split-context partitions and their merge

@pytest.mark.parametrize("P", [16, 64, 512])
def test_partitioned_against_oracle(P):
    wl = _small("f16", 128, 16, lens=[0, 1, 16, 17, 64, 65, 299])
    g = _gpu(wl)
    maxL = int(wl.context_lens.max())
    ws = pa.partition_workspace(wl.num_seqs, wl.num_heads, wl.head_size, maxL, P, DEV)
    out = pa.decode_partitioned(g.q, g.k_cache, g.v_cache, g.block_table, g.context_lens,
                                wl.scale, P, maxL, workspace=ws)
    torch.cuda.synchronize()
    atol, rtol = tol_of(wl)
    a = oracle_arrays(wl)
    ref, parts = oracle.paged_decode_partitioned(a["q"], a["k"], a["v"], a["table"], a["lens"],
                                                 wl.scale, wl.num_kv_heads, 16, "f16", "f16", P)
    assert_close(as_f64(out), ref, atol, rtol, f"merged, P={P}")
    tmp, ml, es = (x.cpu().double().numpy() for x in ws)
    for (s, h), pp in parts.items():
        for p, (m, l, o) in enumerate(pp):
            assert abs(ml[s, h, p] - m) <= 1e-3 + 1e-4 * abs(m), (s, h, p)
            assert abs(es[s, h, p] - l) <= 1e-3 * l, (s, h, p)
            assert_close(tmp[s, h, p], o, atol, rtol, f"partial {(s, h, p)}")


def test_single_partition_equals_one_pass_bit_for_bit():
    wl = _small("bf16", 128, 16)
    g = _gpu(wl)
    maxL = int(wl.context_lens.max())
    one = _decode(g)
    two = pa.decode_partitioned(g.q, g.k_cache, g.v_cache, g.block_table, g.context_lens,
                                wl.scale, 512, maxL)
    torch.cuda.synchronize()
    assert torch.equal(one, two)


# ----------------------------------------------------------------------------
# cache write

def _run_slots(BS):
    """Slot runs of a prefill-like write: an unaligned run across a block
    boundary, an aligned whole quad, a quad with a skipped (-1) token, a quad
    in reversed token order and a lone token."""
    runs = [list(range(5, 5 + 2 * BS + 3)),              # unaligned, crosses blocks
            list(range(4 * BS, 4 * BS + 4)),              # one whole quad
            [5 * BS + 8, 5 * BS + 9, -1, 5 * BS + 11],    # a token skipped inside a quad
            [6 * BS + 3, 6 * BS + 2, 6 * BS + 1, 6 * BS], # reversed order
            [7 * BS + 6]]
    return [x for r in runs for x in r]


def _write_and_compare(slots, cache_fmt, D, BS, KVH, NB, seed, in_fmt=None, sample=None):
    """pa_cache_write of random K/V (in_fmt; default: the cache's 16-bit type,
    f16 for fp8 caches) into a random pool against the oracle's write, both
    caches compared bit for bit.  sample: a seeded fraction of the tokens, the
    only ones the oracle writes, and only their slots are compared (the fp8
    oracle quantises in fp64, one token at a time)."""
    gen = torch.Generator().manual_seed(seed)
    slots = torch.tensor(slots, dtype=torch.int32)
    T = slots.numel()
    in_fmt = in_fmt or ("bf16" if cache_fmt == "bf16" else "f16")
    in_dt = torch.bfloat16 if in_fmt == "bf16" else torch.float16
    k = torch.randn((T, KVH, D), generator=gen).to(in_dt)
    v = torch.randn((T, KVH, D), generator=gen).to(in_dt)
    if cache_fmt == "e4m3fn":
        kc0 = torch.randint(0, 256, (NB, KVH, BS, D), generator=gen, dtype=torch.uint8)
        vc0 = torch.randint(0, 256, (NB, KVH, BS // 4, D, 4), generator=gen, dtype=torch.uint8)
        kc0[(kc0 & 0x7F) == 0x7F] = 0                    # no NaN codes in the pool
        vc0[(vc0 & 0x7F) == 0x7F] = 0
        kc, vc = kc0.view(torch.float8_e4m3fn), vc0.view(torch.float8_e4m3fn)
        ks, vs = 0.5, 0.25
    else:
        kc = torch.randn((NB, KVH, BS, D), generator=gen).to(in_dt)
        vc = torch.randn((NB, KVH, BS // 4, D, 4), generator=gen).to(in_dt)
        ks = vs = 1.0
    gk, gv = kc.to(DEV), vc.to(DEV)
    pa.cache_write(k.to(DEV), v.to(DEV), gk, gv, slots.to(DEV), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    if sample is None:
        ok, ov = oracle.cache_write(to_numpy_bits(k), to_numpy_bits(v), to_numpy_bits(kc),
                                    to_numpy_bits(vc), slots.numpy(), BS, cache_fmt, ks, vs)
        assert to_numpy_bits(gk).tobytes() == ok.tobytes()
        assert to_numpy_bits(gv).tobytes() == ov.tobytes()
        return
    pick = np.random.default_rng(seed).random(T) < sample
    sub = np.where(pick, slots.numpy(), -1)
    ok, ov = oracle.cache_write(to_numpy_bits(k), to_numpy_bits(v), to_numpy_bits(kc),
                                to_numpy_bits(vc), sub, BS, cache_fmt, ks, vs)
    gkn, gvn = to_numpy_bits(gk), to_numpy_bits(gv)
    written = [int(x) for x in sub if x >= 0]
    assert len(written) > 50
    for sl in written:
        b, o = divmod(sl, BS)
        assert gkn[b, :, o].tobytes() == ok[b, :, o].tobytes(), f"K slot {sl}"
        assert gvn[b, :, o // 4, :, o % 4].tobytes() == ov[b, :, o // 4, :, o % 4].tobytes(), \
            f"V slot {sl}"


@pytest.mark.parametrize("cache_fmt,D,BS", [("f16", 128, 16), ("bf16", 64, 32),
                                            ("e4m3fn", 128, 16), ("e4m3fn", 64, 32)])
def test_cache_write_runs_bit_exact(cache_fmt, D, BS):
    """Whole token quads are written four tokens at a time, the rest token by
    token: both against the oracle's write, bit for bit."""
    _write_and_compare(_run_slots(BS), cache_fmt, D, BS, KVH=3, NB=9, seed=11)


def _ragged_chunk_slots(rng, BS, NB, min_tokens):
    """Prefill-like slots over a permuted pool: sequences with a cached prefix
    of any length (chunks start mid-quad and mid-block) and a chunk of 1..90
    tokens, about 1% of tokens skipped (-1), one quad in reversed order, and
    a token count that is not a multiple of 8."""
    perm = rng.permutation(NB).tolist()
    slots = []
    while len(slots) < min_tokens:
        ctx, n = int(rng.integers(0, 40)), int(rng.integers(1, 91))
        nblk = -(-(ctx + n) // BS)
        blocks, perm = perm[:nblk], perm[nblk:]
        assert len(blocks) == nblk, "pool too small"
        slots += [blocks[t // BS] * BS + t % BS for t in range(ctx, ctx + n)]
    slots = np.array(slots, dtype=np.int64)
    slots[rng.random(slots.size) < 0.01] = -1
    q = 4 * int(rng.integers(10, slots.size // 4 - 10))
    slots[q:q + 4] = slots[q:q + 4][::-1].copy()
    if slots.size % 8 == 0:
        slots = slots[:-3]
    return slots.tolist()


@pytest.mark.parametrize("cache_fmt,D,BS", [("f16", 128, 16), ("bf16", 64, 32),
                                            ("e4m3fn", 128, 16)])
def test_cache_write_wide_grid_ragged_bit_exact(cache_fmt, D, BS):
    """A write of 1,100+ tokens over 32 kv heads, enough wavefronts that each
    takes several token quads: groups whose quads are all whole and aligned
    take the load-all-then-store path, the others (a chunk's first or last
    tokens, skips, the reversed quad, the ragged end) the per-token one; both
    against the oracle's write, bit for bit."""
    rng = np.random.default_rng(31)
    KVH, NB = 32, 160 if BS == 16 else 100
    slots = _ragged_chunk_slots(rng, BS, NB, min_tokens=1100)
    T = len(slots)
    assert T % 8 != 0 and -(-T // 8) * KVH >= 4096
    _write_and_compare(slots, cache_fmt, D, BS, KVH=KVH, NB=NB, seed=12)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("BS", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("in_fmt,cache_fmt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3fn"),
                                              ("bf16", "e4m3fn")])
def test_cache_write_every_kernel_bit_exact(in_fmt, cache_fmt, D, BS, wide):
    """Every compiled cache write: input and cache types, head and block
    sizes, one token quad per wavefront (a narrow grid) or several (a wide
    one), with ragged prefill-like slots; bit for bit against the oracle
    (wide fp8 writes: on an eighth of the tokens, drawn at random)."""
    rng = np.random.default_rng(32)
    KVH, NB = (32, 160 if BS == 16 else 100) if wide else (3, 120 if BS == 16 else 70)
    slots = _ragged_chunk_slots(rng, BS, NB, min_tokens=1100 if wide else 300)
    if wide:
        assert -(-len(slots) // 8) * KVH >= 4096
    _write_and_compare(slots, cache_fmt, D, BS, KVH=KVH, NB=NB, seed=13, in_fmt=in_fmt,
                       sample=0.125 if wide and cache_fmt == "e4m3fn" else None)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_cache_write_16bit_bit_exact(dtype):
    wl = workloads.llama7b_mha(seed=9, num_seqs=9, len_range=(0, 100), num_heads=4,
                               dtype=dtype)
    g = _gpu(wl)
    slots = wl.slot_mapping.clone()
    slots[2] = -1
    gs = slots.to(DEV)
    pa.cache_write(g.new_k, g.new_v, g.k_cache, g.v_cache, gs)
    torch.cuda.synchronize()
    a = oracle_arrays(wl)
    kc, vc = oracle.cache_write(to_numpy_bits(wl.new_k), to_numpy_bits(wl.new_v), a["k"], a["v"],
                                slots.numpy(), wl.block_size, dtype)
    assert to_numpy_bits(g.k_cache).tobytes() == kc.tobytes()
    assert to_numpy_bits(g.v_cache).tobytes() == vc.tobytes()
