"""Shared helpers of the GPU parity tests: run the CPU oracle on a workload
and compare element by element."""
import numpy as np
import torch

import oracle
from workloads import to_numpy_bits

# |gpu - oracle| <= atol + rtol * |oracle| per element (16-bit / fp8 caches)
TOL = {"f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "e4m3fn": (5e-3, 1e-2)}


def tol_of(wl):
    return TOL[wl.cache_dtype]


def oracle_arrays(wl):
    return dict(q=to_numpy_bits(wl.q), k=to_numpy_bits(wl.k_cache), v=to_numpy_bits(wl.v_cache),
                table=wl.block_table.cpu().numpy(), lens=wl.context_lens.cpu().numpy())


def oracle_decode(wl, lens=None, seqs=None, heads=None, arrays=None):
    a = arrays or oracle_arrays(wl)
    L = a["lens"] if lens is None else np.asarray(lens, dtype=np.int32)
    return oracle.paged_decode(a["q"], a["k"], a["v"], a["table"], L, wl.scale, wl.num_kv_heads,
                               wl.block_size, wl.q_dtype, wl.cache_dtype, wl.k_scale, wl.v_scale,
                               seqs=seqs, heads=heads)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def assert_close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(ref)), "oracle produced non-finite values"
    assert np.all(np.isfinite(got)), f"{what}: GPU produced non-finite values"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
            f"gpu {got[i]!r} oracle {ref[i]!r}; max abs err {err.max():.3e}, "
            f"max rel err {(err / np.maximum(np.abs(ref), 1e-30)).max():.3e}")
    return float(err.max())


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def sampled_oracle(wl, pairs, lens=None):
    """Oracle outputs out[s, h, :] for the listed (s, h) pairs, reading only
    the blocks of those sequences and the needed kv head (host copies)."""
    import torch as _t
    table = wl.block_table.cpu().numpy()
    L = (wl.context_lens if lens is None else lens).cpu().numpy()
    G = wl.num_heads // wl.num_kv_heads
    res = []
    for s, h in pairs:
        n = oracle.num_logical_blocks(int(L[s]), wl.block_size)
        ids = _t.from_numpy(table[s, :n].astype(np.int64)).to(wl.k_cache.device)
        kvh = h // G
        k = to_numpy_bits(wl.k_cache.index_select(0, ids)[:, kvh:kvh + 1])
        v = to_numpy_bits(wl.v_cache.index_select(0, ids)[:, kvh:kvh + 1])
        q = to_numpy_bits(wl.q[s:s + 1, h:h + 1])
        row = np.arange(max(n, 1), dtype=np.int32)[None, :]
        out = oracle.paged_decode(q, k, v, row, np.array([L[s]], dtype=np.int32), wl.scale, 1,
                                  wl.block_size, wl.q_dtype, wl.cache_dtype, wl.k_scale,
                                  wl.v_scale)
        res.append(out[0, 0])
    return np.stack(res)


def sample_pairs(wl, count, seed=0):
    """(s, h) pairs: the longest and shortest sequences plus random ones."""
    rng = np.random.default_rng(seed)
    L = wl.context_lens.cpu().numpy()
    seqs = [int(np.argmax(L)), int(np.argmin(L))]
    seqs += [int(x) for x in rng.integers(0, wl.num_seqs, count - 2)]
    return [(s, int(rng.integers(0, wl.num_heads))) for s in seqs]


def capture_step_inputs(wl, pairs):
    """Host copies, taken before a decode step runs, of what the oracle needs
    for each (s, h): q row, the blocks of s's cached context for kv head
    h // G, and s's new token."""
    import torch as _t
    table = wl.block_table.cpu().numpy()
    L = wl.context_lens.cpu().numpy()
    G = wl.num_heads // wl.num_kv_heads
    res = []
    for s, h in pairs:
        n = oracle.num_logical_blocks(int(L[s]), wl.block_size)
        ids = _t.from_numpy(table[s, :n].astype(np.int64)).to(wl.k_cache.device)
        kvh = h // G
        res.append(dict(
            s=s, h=h, kvh=kvh, L=int(L[s]), n=n,
            q=to_numpy_bits(wl.q[s:s + 1, h:h + 1]),
            k=to_numpy_bits(wl.k_cache.index_select(0, ids)[:, kvh:kvh + 1]),
            v=to_numpy_bits(wl.v_cache.index_select(0, ids)[:, kvh:kvh + 1]),
            k_new=to_numpy_bits(wl.new_k[s:s + 1, kvh:kvh + 1]),
            v_new=to_numpy_bits(wl.new_v[s:s + 1, kvh:kvh + 1]),
            slot=int(wl.slot_mapping[s])))
    return res


def step_oracle(wl, captured):
    """Oracle outputs of one decode step (new token stored, context L + 1) for
    the captured pairs, and the cache values each new token's slot must hold:
    list of (out [D], k_slot [D], v_slot [D]) with the slot values as raw
    cache bits/codes."""
    res = []
    BS = wl.block_size
    for c in captured:
        row = np.arange(max(c["n"], 1), dtype=np.int32)[None, :]
        nb = max(c["n"], 1)
        k, v = c["k"], c["v"]
        if c["n"] == 0:                     # empty context: one dummy block, never read
            k = np.zeros((1,) + k.shape[1:], dtype=k.dtype)
            v = np.zeros((1,) + v.shape[1:], dtype=v.dtype)
        # the new token goes to the slot after the cached ones inside the
        # gathered sub-pool (one extra block when L fills its blocks)
        off = c["L"] % BS
        blk = c["L"] // BS
        if blk >= nb:
            k = np.concatenate([k, np.zeros_like(k[:1])])
            v = np.concatenate([v, np.zeros_like(v[:1])])
            row = np.arange(blk + 1, dtype=np.int32)[None, :]
        out, kc, vc = oracle.decode_append(
            c["q"], c["k_new"], c["v_new"], k, v, np.array([blk * BS + off], dtype=np.int32), row,
            np.array([c["L"]], dtype=np.int32), wl.scale, 1, BS, wl.q_dtype, wl.cache_dtype,
            wl.k_scale, wl.v_scale)
        res.append((out[0, 0], kc[blk, 0, off], vc[blk, 0, off // 4, :, off % 4]))
    return res
