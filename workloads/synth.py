"""Seeded synthetic inputs for paged decode attention.

Cache layouts produced here (the library's layout, both row-major):
  k_cache [num_blocks, num_kv_heads, block_size, head_size]        token-major tile
  v_cache [num_blocks, num_kv_heads, block_size/4, head_size, 4]   token-quad tile
(token t, head dim d of a V tile sits at [t // 4, d, t % 4]).

Every workload follows one decode step of the vLLM block manager (vLLM paper
summary, section 3 "Decoding"; aivaro.ru "How does paged attention work",
section 4.1): context_lens[s] tokens are already cached, the new token goes to
logical position context_lens[s], and the block table already maps the logical
block that position falls in (a fresh physical block is taken when the last
one is full, as in the data-sketchers "Paged attention" decode example).

Draw order per config (fixed, seed = config index, torch CPU generator unless a
device generator is asked for): context lengths -> [sharing set] -> physical
block permutation -> q -> K pool -> V pool -> new k -> new v.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

TORCH_DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "e4m3fn": torch.float8_e4m3fn,
}


@dataclass
class Workload:
    name: str
    q: torch.Tensor              # [S, H, D]  q_dtype
    k_cache: torch.Tensor        # [NB, KVH, BS, D]  cache_dtype
    v_cache: torch.Tensor        # [NB, KVH, BS/4, D, 4]  cache_dtype
    block_table: torch.Tensor    # [S, MB] int32, -1 = unallocated
    context_lens: torch.Tensor   # [S] int32, tokens already in the cache
    new_k: torch.Tensor          # [S, KVH, D]  q_dtype, the step's new token
    new_v: torch.Tensor          # [S, KVH, D]
    slot_mapping: torch.Tensor   # [S] int32, slot of position context_lens[s]
    scale: float
    num_kv_heads: int
    block_size: int
    q_dtype: str
    cache_dtype: str
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_size: int = 0
    shared_blocks: Sequence[int] = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_size(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def to(self, device) -> "Workload":
        mv = lambda t: t.to(device)
        return replace(
            self, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
            block_table=mv(self.block_table), context_lens=mv(self.context_lens),
            new_k=mv(self.new_k), new_v=mv(self.new_v), slot_mapping=mv(self.slot_mapping))


# ----------------------------------------------------------------------------
# helpers

def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _allocate(cover: Sequence[int], block_size: int, max_blocks: int,
              gen: torch.Generator, shared: Optional[dict] = None,
              spare: int = 1):
    """Block tables whose rows map ceil(cover[s]/block_size) logical blocks.

    shared = {"seqs": [...], "blocks": n} makes those sequences' first n
    logical blocks point at the same n physical blocks (a shared prefix).
    Returns (table[S, MB] int32 with -1 padding, num_blocks, shared_ids).
    """
    S = len(cover)
    need = [-(-int(c) // block_size) for c in cover]
    n_shared = shared["blocks"] if shared else 0
    share_set = set(shared["seqs"]) if shared else set()
    private = sum(n - (n_shared if s in share_set else 0) for s, n in enumerate(need))
    num_blocks = n_shared + private + spare
    perm = torch.randperm(num_blocks, generator=gen, device=gen.device).tolist()
    shared_ids = perm[:n_shared]
    nxt = n_shared
    table = torch.full((S, max_blocks), -1, dtype=torch.int32)
    for s in range(S):
        j0 = 0
        if s in share_set:
            table[s, :n_shared] = torch.tensor(shared_ids, dtype=torch.int32)
            j0 = n_shared
        for j in range(j0, need[s]):
            table[s, j] = perm[nxt]
            nxt += 1
    return table, num_blocks, shared_ids


def _new_token_slots(table: torch.Tensor, ctx: torch.Tensor, block_size: int) -> torch.Tensor:
    """Slot (physical block * block_size + offset) of position ctx[s]."""
    slots = []
    for s, L in enumerate(ctx.tolist()):
        phys = int(table[s, L // block_size])
        slots.append(phys * block_size + L % block_size)
    return torch.tensor(slots, dtype=torch.int32)


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def _assemble(name, ctx, table, num_blocks, gen, device, *, H, KVH, D, BS,
              q_dtype, cache_dtype="", partition_size=0, shared_ids=()):
    cache_dtype = cache_dtype or q_dtype
    S = len(ctx)
    tq = TORCH_DTYPES[q_dtype]
    q = _randn((S, H, D), gen, device, tq)
    k_cache = _randn((num_blocks, KVH, BS, D), gen, device, TORCH_DTYPES[cache_dtype])
    v_cache = _randn((num_blocks, KVH, BS // 4, D, 4), gen, device, TORCH_DTYPES[cache_dtype])
    new_k = _randn((S, KVH, D), gen, device, tq)
    new_v = _randn((S, KVH, D), gen, device, tq)
    ctx_t = torch.tensor(ctx, dtype=torch.int32)
    return Workload(
        name=name, q=q, k_cache=k_cache, v_cache=v_cache,
        block_table=table.to(device), context_lens=ctx_t.to(device),
        new_k=new_k, new_v=new_v,
        slot_mapping=_new_token_slots(table, ctx_t, BS).to(device),
        scale=float(np.float32(1.0 / math.sqrt(D))), num_kv_heads=KVH, block_size=BS,
        q_dtype=q_dtype, cache_dtype=cache_dtype, partition_size=partition_size,
        shared_blocks=list(shared_ids))


def _uniform_lengths(gen, S, lo, hi, lengths=None):
    drawn = torch.randint(lo, hi + 1, (S,), generator=gen, device=gen.device).cpu().tolist()
    if lengths is None:
        return drawn
    # explicit lengths (tests of edge cases) replace the first len(lengths) draws
    lengths = [int(x) for x in lengths]
    assert len(lengths) <= S and all(0 <= x <= hi for x in lengths)
    return lengths + drawn[len(lengths):]


# ----------------------------------------------------------------------------
# the five workloads (full sizes by default; keyword overrides shrink them)

def worked_example(seed: int = 0, device: str = "cpu") -> Workload:
    """data-sketchers.com "Paged attention", decode-path example: three
    sequences with cache_seqlens [30, 32, 70], block size 32, at most 4 blocks
    per sequence and the page's block table.  Heads, head size and dtype are
    the benchmark definition's (4 = 4 kv heads, head size 64, fp16 N(0,1))."""
    gen = _gen(seed, device)
    ctx = [30, 32, 70]
    table = torch.tensor([[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]], dtype=torch.int32)
    return _assemble("worked_example", ctx, table, 8, gen, device,
                     H=4, KVH=4, D=64, BS=32, q_dtype="f16")


def llama7b_mha(seed: int = 1, device: str = "cpu", num_seqs: int = 64,
                len_range=(128, 2048), num_heads: int = 32, head_size: int = 128,
                block_size: int = 16, dtype: str = "f16", lengths=None) -> Workload:
    """Llama-7B-shaped MHA decode layer: 64 sequences, 32 heads = 32 kv heads,
    head size 128, block size 16, context lengths uniform in [128, 2048],
    randomly permuted physical blocks, fp16 N(0,1)."""
    gen = _gen(seed, device)
    ctx = _uniform_lengths(gen, num_seqs, *len_range, lengths=lengths)
    mb = -(-(len_range[1] + 1) // block_size)
    table, nb, _ = _allocate([c + 1 for c in ctx], block_size, mb, gen)
    return _assemble("llama7b_mha", ctx, table, nb, gen, device, H=num_heads,
                     KVH=num_heads, D=head_size, BS=block_size, q_dtype=dtype)


def gqa(seed: int = 2, device: str = "cpu", num_seqs: int = 128, len_range=(512, 4096),
        num_heads: int = 64, num_kv_heads: int = 8, head_size: int = 128,
        block_size: int = 16, dtype: str = "bf16", lengths=None) -> Workload:
    """GQA decode: 128 sequences, 64 query heads over 8 kv heads, head size
    128, block size 16, context lengths uniform in [512, 4096], bf16 N(0,1)."""
    gen = _gen(seed, device)
    ctx = _uniform_lengths(gen, num_seqs, *len_range, lengths=lengths)
    mb = -(-(len_range[1] + 1) // block_size)
    table, nb, _ = _allocate([c + 1 for c in ctx], block_size, mb, gen)
    return _assemble("gqa", ctx, table, nb, gen, device, H=num_heads, KVH=num_kv_heads,
                     D=head_size, BS=block_size, q_dtype=dtype)


def long_context(seed: int = 3, device: str = "cpu", num_seqs: int = 8,
                 len_range=(32768, 131072), num_heads: int = 32, head_size: int = 128,
                 block_size: int = 16, partition_size: int = 512,
                 dtype: str = "f16", lengths=None) -> Workload:
    """Long-context partitioned decode: 8 sequences, 32 heads = 32 kv heads,
    head size 128, block size 16, context lengths uniform in [32768, 131072],
    fp16 N(0,1), 512-token partitions.  The full-size pool is ~10.7 GB: draw
    it with device="cuda"."""
    gen = _gen(seed, device)
    ctx = _uniform_lengths(gen, num_seqs, *len_range, lengths=lengths)
    mb = -(-(len_range[1] + 1) // block_size)
    table, nb, _ = _allocate([c + 1 for c in ctx], block_size, mb, gen)
    return _assemble("long_context", ctx, table, nb, gen, device, H=num_heads,
                     KVH=num_heads, D=head_size, BS=block_size, q_dtype=dtype,
                     partition_size=partition_size)


def fp8_shared_prefix(seed: int = 4, device: str = "cpu", num_seqs: int = 256,
                      median: float = 1024.0, sigma: float = 1.0, cap: int = 8192,
                      num_heads: int = 64, num_kv_heads: int = 8, head_size: int = 128,
                      block_size: int = 16, prefix_tokens: int = 512,
                      share_fraction: float = 0.25) -> Workload:
    """fp8 KV cache with shared prefixes: 256 sequences, 64 query heads over 8
    kv heads, head size 128, block size 16, e4m3fn K/V with one fp32 scale per
    cache, context lengths lognormal (median 1024, capped at 8192), a quarter
    of the sequences sharing one 512-token prefix through the same physical
    blocks (parallel sampling of one prompt), q and new k/v in bf16.

    Reading taken: sigma = 1; lengths round(exp(N(ln median, sigma))) clipped
    to [1, cap]; the sharing sequences are the first share_fraction*S of a
    random permutation restricted to lengths >= prefix_tokens.  Pool values
    are N(0,1) fp32 coded as e4m3fn(value / scale) with scale = amax / 448
    over the pool and the new tokens, so nothing saturates; the coding uses
    torch's own float8 cast."""
    assert prefix_tokens % block_size == 0
    gen = _gen(seed, device)
    z = torch.randn((num_seqs,), generator=gen, device=device, dtype=torch.float64).cpu()
    ctx = torch.clamp(torch.round(torch.exp(z * sigma + math.log(median))), 1, cap)
    ctx = [int(c) for c in ctx.tolist()]
    order = torch.randperm(num_seqs, generator=gen, device=device).cpu().tolist()
    n_share = int(round(share_fraction * num_seqs))
    share = [s for s in order if ctx[s] >= prefix_tokens][:n_share]
    mb = -(-(cap + 1) // block_size)
    table, nb, shared_ids = _allocate(
        [c + 1 for c in ctx], block_size, mb, gen,
        shared={"seqs": share, "blocks": prefix_tokens // block_size})
    S, H, KVH, D, BS = num_seqs, num_heads, num_kv_heads, head_size, block_size
    q = _randn((S, H, D), gen, device, torch.bfloat16)
    k32 = torch.randn((nb, KVH, BS, D), generator=gen, device=device, dtype=torch.float32)
    v32 = torch.randn((nb, KVH, BS // 4, D, 4), generator=gen, device=device, dtype=torch.float32)
    new_k = _randn((S, KVH, D), gen, device, torch.bfloat16)
    new_v = _randn((S, KVH, D), gen, device, torch.bfloat16)
    k_amax = max(float(k32.abs().max()), float(new_k.float().abs().max()))
    v_amax = max(float(v32.abs().max()), float(new_v.float().abs().max()))
    k_scale = float(np.float32(k_amax / 448.0))
    v_scale = float(np.float32(v_amax / 448.0))
    k_inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(k_scale, dtype=torch.float32)
    v_inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(v_scale, dtype=torch.float32)
    k_cache = (k32 * k_inv.to(device)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    del k32
    v_cache = (v32 * v_inv.to(device)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    del v32
    ctx_t = torch.tensor(ctx, dtype=torch.int32)
    return Workload(
        name="fp8_shared_prefix", q=q, k_cache=k_cache, v_cache=v_cache,
        block_table=table.to(device), context_lens=ctx_t.to(device), new_k=new_k,
        new_v=new_v, slot_mapping=_new_token_slots(table, ctx_t, BS).to(device),
        scale=float(np.float32(1.0 / math.sqrt(D))), num_kv_heads=KVH, block_size=BS,
        q_dtype="bf16", cache_dtype="e4m3fn", k_scale=k_scale, v_scale=v_scale,
        shared_blocks=shared_ids)


CONFIGS = {
    "worked_example": worked_example,
    "llama7b_mha": llama7b_mha,
    "gqa": gqa,
    "long_context": long_context,
    "fp8_shared_prefix": fp8_shared_prefix,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)


# ----------------------------------------------------------------------------
# test helpers (no arithmetic of the method)

def poison_unused_slots(wl: Workload, covered: Optional[Sequence[int]] = None,
                        value: float = float("nan")) -> Workload:
    """Fill every cache slot that no sequence's first covered[s] tokens use
    with `value` (NaN by default; for e4m3fn the NaN code 0x7F).  Returns a
    new workload; the input tensors are not modified."""
    cov = wl.context_lens.cpu().tolist() if covered is None else list(covered)
    BS = wl.block_size
    used = torch.zeros((wl.num_blocks, BS), dtype=torch.bool)
    table = wl.block_table.cpu()
    for s, L in enumerate(cov):
        for t in range(L):
            used[int(table[s, t // BS]), t % BS] = True
    dev = wl.k_cache.device
    k = wl.k_cache.clone()
    v = wl.v_cache.clone()
    unused = (~used).to(dev)
    unused_v = unused.view(wl.num_blocks, BS // 4, 1, 4)[:, None]     # [NB, 1, BS/4, 1, 4]
    if wl.cache_dtype == "e4m3fn":
        kb, vb = k.view(torch.uint8), v.view(torch.uint8)
        code = 0x7F if value != value else int(torch.tensor(value).to(torch.float8_e4m3fn).view(torch.uint8))
        kb.masked_fill_(unused[:, None, :, None], code)
        vb.masked_fill_(unused_v, code)
    else:
        k.masked_fill_(unused[:, None, :, None], value)
        v.masked_fill_(unused_v, value)
    return replace(wl, k_cache=k, v_cache=v)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Raw values for the CPU oracle: float16 -> np.float16, bfloat16 -> its
    uint16 bit patterns, float8_e4m3fn -> its uint8 codes, ints unchanged."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float16:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
