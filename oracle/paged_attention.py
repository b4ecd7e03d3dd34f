"""Plain fp64 CPU oracle of paged decode attention and of the KV cache write.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, and where the pages define it:

* Paged KV cache.  The K/V vectors of a sequence live in fixed-size blocks of
  `block_size` tokens; a per-sequence block table maps logical block j (tokens
  j*BS .. j*BS+BS-1) to a physical block of the pool; -1 marks an unallocated
  entry.  ("How does paged attention work (in detail)", section 2 and 4.1;
  "Paged attention" wiki, decode-path example; vLLM paper summary, section 2.)
* Cache layouts (this library's; the pages do not fix one):
  k_cache [NB, KVH, BS, D]: a tile is token-major;
  v_cache [NB, KVH, BS/4, D, 4]: a tile holds, for each group of 4
  consecutive tokens, the D head dims, each with those 4 tokens' values
  (token t, dim d at [t // 4, d, t % 4]).
* Scores: x_t = scale * <q, k_t> over the whole head ("Paged Attention" design
  page, section "QK").
* Softmax: m = max_t x_t, f_t = exp(x_t - m), l = sum_t f_t, p = f / l
  (design page, section "Softmax", the displayed formula).
* Tokens at positions >= context_len do not take part (design page, section
  "Softmax", qk_max and logits: the mask token_idx >= context_len).
* Output: out = sum_t p_t * v_t (design page, sections "Value" and "LV").
* Query head h reads kv head h // (H / KVH) (contiguous groups; the pages only
  name num_kv_heads / kv_head_idx).

Readings where the pages are silent (each also listed in the design notes):
  - context_lens counts the tokens attended; the new token of a decode step is
    written first and attended with context_len + 1.
  - the 1e-6 added to the exp sum on the design page is not part of the
    definition (l >= 1 always, since the max term is e^0).
  - an empty context gives a zero output.
  - a partition p of P tokens yields (m_p, l_p, o_p) with o_p normalised;
    merging uses M = max m_p, l = sum l_p e^(m_p - M),
    out = sum (l_p e^(m_p - M) / l) o_p.  This is the softmax definition
    split over disjoint token sets; the pages do not describe the merge.
  - a block id outside [0, num_blocks) inside the context, or a context
    longer than the table, is a caller error (ValueError here).
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .formats import quantise_e4m3fn, to_f64


# ----------------------------------------------------------------------------
# indexing (block table -> slots)

def num_logical_blocks(context_len: int, block_size: int) -> int:
    """Logical blocks holding context_len tokens: ceil(L / BS)."""
    return -(-int(context_len) // int(block_size))


def validate(block_table: np.ndarray, context_lens: np.ndarray, block_size: int,
             num_blocks: int, num_heads: int = 1, num_kv_heads: int = 1) -> None:
    """Raise ValueError on inputs the method leaves undefined."""
    if num_kv_heads <= 0 or num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    S, MB = block_table.shape
    if context_lens.shape != (S,):
        raise ValueError("context_lens must have one entry per sequence")
    for s in range(S):
        L = int(context_lens[s])
        if L < 0 or L > MB * block_size:
            raise ValueError(f"sequence {s}: context length {L} outside [0, {MB * block_size}]")
        for j in range(num_logical_blocks(L, block_size)):
            b = int(block_table[s, j])
            if b < 0 or b >= num_blocks:
                raise ValueError(f"sequence {s}: logical block {j} maps to {b}, "
                                 f"not a block of the pool [0, {num_blocks})")


def token_slots(block_table_row: np.ndarray, context_len: int, block_size: int
                ) -> List[Tuple[int, int]]:
    """(physical block, offset in block) of logical positions 0..L-1:
    position t sits in logical block t // BS at offset t % BS ("How does paged
    attention work", section 4.1, steps 2 and 5)."""
    return [(int(block_table_row[t // block_size]), t % block_size)
            for t in range(int(context_len))]


def next_slot(block_table_row: np.ndarray, context_len: int, block_size: int) -> int:
    """Slot of the token written at position context_len: the physical block
    that logical block context_len // BS maps to, times BS, plus the offset
    context_len % BS.  Raises if that logical block is unallocated (the block
    manager must map it first, as in the vLLM paper summary's second decode
    step)."""
    j = int(context_len) // block_size
    if j >= len(block_table_row) or int(block_table_row[j]) < 0:
        raise ValueError("logical block of the new token is not allocated")
    return int(block_table_row[j]) * block_size + int(context_len) % block_size


# ----------------------------------------------------------------------------
# gather + attention

def v_tiles_to_rows(vt: np.ndarray) -> np.ndarray:
    """V tiles [n, BS/4, D, 4] -> rows [n * BS, D] in token order."""
    n, q4, D, four = vt.shape
    return np.transpose(vt, (0, 1, 3, 2)).reshape(n * q4 * four, D)


def softmax_stats(x: np.ndarray):
    """(m, l, p) of the design page's softmax definition."""
    m = np.max(x)
    f = np.exp(x - m)
    l = np.sum(f)
    return m, l, f / l


def _dequant(cache: np.ndarray, fmt: str, scale: float) -> np.ndarray:
    c = to_f64(cache, fmt)
    if fmt == "e4m3fn":
        c = c * np.float64(np.float32(scale))
    return c


def _chunk_cache(cache, fmt, scale, ids, kv_head):
    """Dequantised tiles of the listed physical blocks for one kv head."""
    return _dequant(np.ascontiguousarray(cache[ids, kv_head]), fmt, scale)


def decode_sequence(q_s: np.ndarray, k_cache, v_cache, table_row, context_len: int,
                    scale: float, num_kv_heads: int, block_size: int, cache_fmt: str,
                    k_scale: float = 1.0, v_scale: float = 1.0,
                    heads=None, return_probs: bool = False):
    """Decode attention of one sequence.  q_s is fp64 [H, D]; the caches are
    raw arrays in cache_fmt.  Returns out [len(heads), D] fp64 (and the
    softmax weights per head when return_probs)."""
    H, D = q_s.shape
    G = H // num_kv_heads
    heads = range(H) if heads is None else heads
    L = int(context_len)
    nblk = num_logical_blocks(L, block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64)
    out = np.zeros((len(heads), D), dtype=np.float64)
    probs = []
    cached = {}
    for i, h in enumerate(heads):
        if L == 0:
            probs.append(np.zeros(0))
            continue
        kvh = h // G
        if kvh not in cached:
            Kt = _chunk_cache(k_cache, cache_fmt, k_scale, ids, kvh)      # [nblk, BS, D]
            Vt = _chunk_cache(v_cache, cache_fmt, v_scale, ids, kvh)      # [nblk, BS/4, D, 4]
            K = Kt.reshape(nblk * block_size, D)[:L]
            V = v_tiles_to_rows(Vt)[:L]
            cached = {kvh: (K, V)}
        K, V = cached[kvh]
        x = np.float64(np.float32(scale)) * (K @ q_s[h])
        _, _, p = softmax_stats(x)
        out[i] = p @ V
        probs.append(p)
    return (out, probs) if return_probs else out


def paged_decode(q, k_cache, v_cache, block_table, context_lens, scale: float,
                 num_kv_heads: int, block_size: int, q_fmt: str, cache_fmt: str,
                 k_scale: float = 1.0, v_scale: float = 1.0, seqs=None, heads=None):
    """out[s, h, :] for every (or the listed) sequence and head, fp64.

    q [S, H, D] raw in q_fmt; caches raw in cache_fmt; block_table [S, MB]
    int32; context_lens [S] int32."""
    S, H, D = q.shape
    NB = k_cache.shape[0]
    seqs = list(range(S)) if seqs is None else list(seqs)
    validate(block_table[seqs], context_lens[seqs], block_size, NB, H, num_kv_heads)
    hs = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(seqs), len(hs), D), dtype=np.float64)
    for i, s in enumerate(seqs):
        q_s = to_f64(q[s], q_fmt)
        out[i] = decode_sequence(q_s, k_cache, v_cache, block_table[s], int(context_lens[s]),
                                 scale, num_kv_heads, block_size, cache_fmt,
                                 k_scale, v_scale, heads=hs)
    return out


# ----------------------------------------------------------------------------
# split-context partitions and their merge

def partition_partials(q_s: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       partition_size: int):
    """(m_p, l_p, o_p) over tokens [p*P, min((p+1)*P, L)) for one head;
    q_s [D], K, V [L, D] fp64."""
    L = K.shape[0]
    x = np.float64(np.float32(scale)) * (K @ q_s)
    res = []
    for start in range(0, L, partition_size):
        xs = x[start:start + partition_size]
        m, l, p = softmax_stats(xs)
        res.append((m, l, p @ V[start:start + partition_size]))
    return res


def merge_partials(partials) -> np.ndarray:
    """Merge (m_p, l_p, o_p) triples: M = max m_p, l = sum l_p e^(m_p - M),
    out = sum (l_p e^(m_p - M) / l) o_p.  Empty -> None (caller writes 0)."""
    if not partials:
        return None
    M = max(m for m, _, _ in partials)
    w = [l * math.exp(m - M) for m, l, _ in partials]
    total = sum(w)
    return sum((wi / total) * o for wi, (_, _, o) in zip(w, partials))


def paged_decode_partitioned(q, k_cache, v_cache, block_table, context_lens, scale,
                             num_kv_heads, block_size, q_fmt, cache_fmt, partition_size,
                             k_scale=1.0, v_scale=1.0, seqs=None, heads=None):
    """Per-partition triples and merged output.

    Returns (out [S', H', D], partials) where partials[(s, h)] is the list of
    (m_p, l_p, o_p) in partition order."""
    S, H, D = q.shape
    if partition_size <= 0 or partition_size % block_size != 0:
        raise ValueError("partition size must be a positive multiple of the block size")
    seqs = list(range(S)) if seqs is None else list(seqs)
    validate(block_table[seqs], context_lens[seqs], block_size, k_cache.shape[0], H, num_kv_heads)
    G = H // num_kv_heads
    hs = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(seqs), len(hs), D), dtype=np.float64)
    parts = {}
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        q_s = to_f64(q[s], q_fmt)
        nblk = num_logical_blocks(L, block_size)
        ids = np.asarray(block_table[s, :nblk], dtype=np.int64)
        for j, h in enumerate(hs):
            kvh = h // G
            Kt = _chunk_cache(k_cache, cache_fmt, k_scale, ids, kvh)
            Vt = _chunk_cache(v_cache, cache_fmt, v_scale, ids, kvh)
            K = Kt.reshape(nblk * block_size, D)[:L]
            V = v_tiles_to_rows(Vt)[:L]
            pp = partition_partials(q_s[h], K, V, scale, partition_size)
            parts[(s, h)] = pp
            merged = merge_partials(pp)
            if merged is not None:
                out[i, j] = merged
    return out, parts


# ----------------------------------------------------------------------------
# cache write

def cache_write(k, v, k_cache, v_cache, slot_mapping, block_size: int, cache_fmt: str,
                k_scale: float = 1.0, v_scale: float = 1.0):
    """New caches after writing token i's K/V [KVH, D] to slot slot_mapping[i].

    slot = physical block * BS + offset ("How does paged attention work",
    section 4.1, step 5: the token's K/V goes to its position inside the
    physical block); slot < 0 is skipped.  16-bit caches take the input bits
    unchanged; an e4m3fn cache takes e4m3fn(clamp(fp32(x) * fp32(1/scale)))
    (formats.quantise_e4m3fn).  Inputs are not modified."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    NB = kc.shape[0]
    seen = set()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        if slot in seen:
            raise ValueError(f"slot {slot} written twice")
        seen.add(slot)
        b, o = divmod(int(slot), block_size)
        if b >= NB:
            raise ValueError(f"slot {slot} is outside the pool")
        if cache_fmt == "e4m3fn":
            kk = quantise_e4m3fn(to_f64(k[i], _fmt_of(k)), k_scale)
            vv = quantise_e4m3fn(to_f64(v[i], _fmt_of(v)), v_scale)
        else:
            kk, vv = k[i], v[i]
        kc[b, :, o, :] = kk
        vc[b, :, o // 4, :, o % 4] = vv
    return kc, vc


# ----------------------------------------------------------------------------
# one decode step: cache write and attention in one call

def stored_rows(x, cache_fmt: str, scale: float = 1.0) -> np.ndarray:
    """fp64 values a cache of cache_fmt holds for new rows x (f16 or bf16
    bits), dequantised: 16-bit caches keep the input; e4m3fn caches hold
    quantise_e4m3fn(x, scale), read back times scale."""
    xf = to_f64(x, _fmt_of(x))
    if cache_fmt != "e4m3fn":
        return xf
    codes = quantise_e4m3fn(xf, scale)
    return _dequant(codes, cache_fmt, scale)


def decode_append(q, k, v, k_cache, v_cache, slot_mapping, block_table, context_lens,
                  scale: float, num_kv_heads: int, block_size: int, q_fmt: str, cache_fmt: str,
                  k_scale: float = 1.0, v_scale: float = 1.0, seqs=None):
    """One decode step ("How does paged attention work (in detail)", section
    4.1: the new token's K/V is stored in its slot and the query attends over
    the context including it; vLLM paper summary, section 3 "Decoding").

    Sequence s attends over its cached positions 0 .. L-1 (through the block
    table) followed by its new token k[s], v[s] ([KVH, D]) with the values
    the cache stores for them.  Returns (out [S', H, D] fp64, new k_cache,
    new v_cache), the caches as cache_write leaves them."""
    S, H, D = q.shape
    seqs = list(range(S)) if seqs is None else list(seqs)
    validate(block_table[seqs], context_lens[seqs], block_size, k_cache.shape[0], H, num_kv_heads)
    G = H // num_kv_heads
    kc, vc = cache_write(k, v, k_cache, v_cache, slot_mapping, block_size, cache_fmt,
                         k_scale, v_scale)
    out = np.zeros((len(seqs), H, D), dtype=np.float64)
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        q_s = to_f64(q[s], q_fmt)
        ids = np.asarray(block_table[s, :num_logical_blocks(L, block_size)], dtype=np.int64)
        k_new = stored_rows(k[s], cache_fmt, k_scale)            # [KVH, D]
        v_new = stored_rows(v[s], cache_fmt, v_scale)
        for h in range(H):
            kvh = h // G
            Kt = _chunk_cache(k_cache, cache_fmt, k_scale, ids, kvh)
            Vt = _chunk_cache(v_cache, cache_fmt, v_scale, ids, kvh)
            K = np.concatenate([Kt.reshape(-1, D)[:L], k_new[kvh][None]])
            V = np.concatenate([v_tiles_to_rows(Vt)[:L], v_new[kvh][None]])
            x = np.float64(np.float32(scale)) * (K @ q_s[h])
            _, _, p = softmax_stats(x)
            out[i, h] = p @ V
    return out, kc, vc


# ----------------------------------------------------------------------------
# varlen / chunked prefill over the paged cache

def request_index(cu_seqlens) -> list:
    """Request that each packed token belongs to, from cumulative lengths
    (batching wiki, Varlen path: cu_seq_lens assigns tokens to sequences)."""
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cumulative lengths must start at 0 and not decrease")
    return [r for r in range(len(cu) - 1) for _ in range(cu[r + 1] - cu[r])]


def paged_prefill(q, k_cache, v_cache, block_table, cu_seqlens_q, context_lens, scale: float,
                  num_kv_heads: int, block_size: int, q_fmt: str, cache_fmt: str,
                  k_scale: float = 1.0, v_scale: float = 1.0, causal: bool = True, seqs=None):
    """Attention of several new query tokens per sequence over its paged K/V.

    q [total_q, H, D] packs the sequences' query tokens by cu_seqlens_q
    (batching wiki, Varlen path); sequence s has n_s = cu[s+1] - cu[s] of them
    and context_lens[s] = K_s tokens in the cache, read through its block
    table.  The queries are the sequence's last n_s positions (a prefill chunk
    whose K/V were written first): query i sits at position K_s - n_s + i and,
    causal, attends keys 0 .. K_s - n_s + i; otherwise all K_s keys.  A query
    with no key gets zeros.  Returns out [total_q, H, D] fp64 (rows of
    sequences not listed in seqs stay zero)."""
    T, H, D = q.shape
    cu = [int(x) for x in cu_seqlens_q]
    request_index(cu)
    S = len(cu) - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens_q does not cover q")
    seqs = list(range(S)) if seqs is None else list(seqs)
    validate(block_table[seqs], context_lens[seqs], block_size, k_cache.shape[0], H, num_kv_heads)
    G = H // num_kv_heads
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in seqs:
        Ks = int(context_lens[s])
        n = cu[s + 1] - cu[s]
        ids = np.asarray(block_table[s, :num_logical_blocks(Ks, block_size)], dtype=np.int64)
        for kvh in range(num_kv_heads):
            K = _chunk_cache(k_cache, cache_fmt, k_scale, ids, kvh).reshape(-1, D)[:Ks]
            V = v_tiles_to_rows(_chunk_cache(v_cache, cache_fmt, v_scale, ids, kvh))[:Ks]
            for i in range(n):
                last = Ks - n + i if causal else Ks - 1        # last key attended
                if last < 0:
                    continue
                for h in range(kvh * G, (kvh + 1) * G):
                    qv = to_f64(q[cu[s] + i, h], q_fmt)
                    x = np.float64(np.float32(scale)) * (K[:last + 1] @ qv)
                    _, _, p = softmax_stats(x)
                    out[cu[s] + i, h] = p @ V[:last + 1]
    return out


def _fmt_of(a: np.ndarray) -> str:
    if a.dtype == np.float16:
        return "f16"
    if a.dtype == np.uint16:
        return "bf16"
    raise ValueError("new k/v must be f16 (np.float16) or bf16 (uint16 bits)")
