"""Seeded synthetic chunked-prefill batches over a paged cache.

A batch holds, per sequence, ctx_s tokens already cached and a chunk of q_s
new tokens: their queries (packed by cu_seqlens_q, as on the batching wiki's
Varlen path), their K/V (to be written to their slots first) and the block
table covering all ctx_s + q_s tokens.  Draws only; no attention arithmetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Sequence

import numpy as np
import torch

from .synth import TORCH_DTYPES


@dataclass
class PrefillBatch:
    name: str
    q: torch.Tensor              # [T, H, D] q_dtype, packed by cu_seqlens_q
    k_cache: torch.Tensor        # [NB, KVH, BS, D] cache_dtype (chunk slots not yet written)
    v_cache: torch.Tensor        # [NB, KVH, BS/4, D, 4]
    block_table: torch.Tensor    # [S, MB] int32
    cu_seqlens_q: torch.Tensor   # [S + 1] int32
    context_lens: torch.Tensor   # [S] int32, ctx_s + q_s (after the chunk is written)
    new_k: torch.Tensor          # [T, KVH, D] q_dtype, the chunk's K
    new_v: torch.Tensor          # [T, KVH, D]
    slot_mapping: torch.Tensor   # [T] int32, slots of positions ctx_s .. ctx_s + q_s - 1
    scale: float
    num_kv_heads: int
    block_size: int
    q_dtype: str
    cache_dtype: str
    max_seqlen_q: int
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_size(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def to(self, device) -> "PrefillBatch":
        mv = lambda t: t.to(device)
        return replace(self, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
                       block_table=mv(self.block_table), cu_seqlens_q=mv(self.cu_seqlens_q),
                       context_lens=mv(self.context_lens), new_k=mv(self.new_k),
                       new_v=mv(self.new_v), slot_mapping=mv(self.slot_mapping))


def prefill_batch(seed: int, q_lens: Sequence[int], ctx_lens: Sequence[int], num_heads: int,
                  num_kv_heads: int, head_size: int, block_size: int, q_dtype: str = "f16",
                  cache_dtype: str = "", device: str = "cpu", name: str = "prefill",
                  spare_blocks: int = 2) -> PrefillBatch:
    """Sequences with ctx_lens[s] cached tokens and a chunk of q_lens[s] new
    tokens; physical blocks are a random permutation of the pool; values
    N(0,1) (fp8 caches: e4m3fn codes of x / scale with scale = amax / 448
    over the pool and the chunk, from torch's float8 cast)."""
    cache_dtype = cache_dtype or q_dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    S, H, KVH, D, BS = len(q_lens), num_heads, num_kv_heads, head_size, block_size
    total = [int(c) + int(n) for c, n in zip(ctx_lens, q_lens)]
    need = [-(-t // BS) for t in total]
    nb = sum(need) + spare_blocks
    perm = torch.randperm(nb, generator=gen, device=device).cpu().tolist()
    mb = max(max(need), 1)
    table = torch.full((S, mb), -1, dtype=torch.int32)
    used = 0
    for s, n in enumerate(need):
        table[s, :n] = torch.tensor(perm[used:used + n], dtype=torch.int32)
        used += n
    cu = torch.tensor(np.cumsum([0] + [int(n) for n in q_lens]), dtype=torch.int32)
    T = int(cu[-1])
    slots = []
    for s in range(S):
        for t in range(int(ctx_lens[s]), total[s]):
            slots.append(int(table[s, t // BS]) * BS + t % BS)
    tq = TORCH_DTYPES[q_dtype]
    q = torch.randn((T, H, D), generator=gen, device=device, dtype=torch.float32).to(tq)
    k32 = torch.randn((nb, KVH, BS, D), generator=gen, device=device, dtype=torch.float32)
    v32 = torch.randn((nb, KVH, BS // 4, D, 4), generator=gen, device=device, dtype=torch.float32)
    new_k = torch.randn((T, KVH, D), generator=gen, device=device, dtype=torch.float32).to(tq)
    new_v = torch.randn((T, KVH, D), generator=gen, device=device, dtype=torch.float32).to(tq)
    k_scale = v_scale = 1.0
    if cache_dtype == "e4m3fn":
        k_scale = float(np.float32(max(float(k32.abs().max()), float(new_k.float().abs().max())) / 448.0))
        v_scale = float(np.float32(max(float(v32.abs().max()), float(new_v.float().abs().max())) / 448.0))
        ki = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(k_scale, dtype=torch.float32)
        vi = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(v_scale, dtype=torch.float32)
        k_cache = (k32 * ki.to(device)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        v_cache = (v32 * vi.to(device)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    else:
        k_cache = k32.to(TORCH_DTYPES[cache_dtype])
        v_cache = v32.to(TORCH_DTYPES[cache_dtype])
    return PrefillBatch(
        name=name, q=q, k_cache=k_cache, v_cache=v_cache, block_table=table.to(device),
        cu_seqlens_q=cu.to(device), context_lens=torch.tensor(total, dtype=torch.int32).to(device),
        new_k=new_k, new_v=new_v, slot_mapping=torch.tensor(slots, dtype=torch.int32).to(device),
        scale=float(np.float32(1.0 / math.sqrt(D))), num_kv_heads=KVH, block_size=BS,
        q_dtype=q_dtype, cache_dtype=cache_dtype, max_seqlen_q=max([int(n) for n in q_lens] + [0]),
        k_scale=k_scale, v_scale=v_scale)


def llama7b_prefill_chunks(seed: int = 6, device: str = "cpu", num_seqs: int = 16,
                           chunk: int = 512, max_cached: int = 1536) -> PrefillBatch:
    """Chunked prefill on the Llama-7B shape (32 heads = 32 kv heads, head
    128, block 16, fp16): num_seqs sequences, each a chunk of `chunk` new
    tokens after a cached prefix of U{0..max_cached} tokens (a multiple of
    16, as chunks of earlier steps leave it)."""
    gen = torch.Generator().manual_seed(seed)
    ctx = (torch.randint(0, max_cached // 16 + 1, (num_seqs,), generator=gen) * 16).tolist()
    return prefill_batch(seed, [chunk] * num_seqs, ctx, 32, 32, 128, 16, "f16", device=device,
                         name="llama7b_prefill_chunks")


def llama7b_prefill_long(seed: int = 7, device: str = "cpu", num_seqs: int = 8,
                         prompt: int = 4096) -> PrefillBatch:
    """Whole-prompt prefill on the Llama-7B shape (32 heads = 32 kv heads,
    head 128, block 16, fp16): num_seqs prompts of `prompt` tokens with no
    cached prefix, each token attending the prompt up to itself."""
    return prefill_batch(seed, [prompt] * num_seqs, [0] * num_seqs, 32, 32, 128, 16, "f16",
                         device=device, name="llama7b_prefill_long")


def poison_prefill(b: PrefillBatch, covered=None, value: float = float("nan")) -> PrefillBatch:
    """Fill every cache slot outside the sequences' first covered[s] tokens
    (default: their cached prefixes, so the chunk's own slots too) with NaN
    (fp8: code 0x7F)."""
    BS = b.block_size
    table = b.block_table.cpu()
    cu = b.cu_seqlens_q.cpu()
    if covered is None:
        covered = [int(b.context_lens[s]) - int(cu[s + 1] - cu[s]) for s in range(b.num_seqs)]
    used = torch.zeros((b.num_blocks, BS), dtype=torch.bool)
    for s in range(b.num_seqs):
        for t in range(int(covered[s])):
            used[int(table[s, t // BS]), t % BS] = True
    dev = b.k_cache.device
    k, v = b.k_cache.clone(), b.v_cache.clone()
    unused = (~used).to(dev)
    unused_v = unused.view(b.num_blocks, BS // 4, 1, 4)[:, None]
    if b.cache_dtype == "e4m3fn":
        k.view(torch.uint8).masked_fill_(unused[:, None, :, None], 0x7F)
        v.view(torch.uint8).masked_fill_(unused_v, 0x7F)
    else:
        k.masked_fill_(unused[:, None, :, None], value)
        v.masked_fill_(unused_v, value)
    return replace(b, k_cache=k, v_cache=v)
