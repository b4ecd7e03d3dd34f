"""The five decode workloads and the chunked-prefill workload at full size,
in the launch configuration bench.py
times (one decode step: the new tokens stored and attention over
context_len + 1; one launch of pa_decode_append for the one-pass workloads,
pa_cache_write + pa_decode_partitioned + pa_reduce for the long-context one),
checked against the oracle on sampled (sequence, head) outputs and on the
sampled sequences' written slots; the whole output is checked for
finiteness.  The oracle's inputs are host copies taken before the step."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_78_amd as pa
import workloads
from gpu_helpers import (as_f64, assert_close, capture_step_inputs, oracle_arrays, sample_pairs,
                         step_oracle, tol_of)
from workloads import to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _step(wl):
    if wl.partition_size:
        pa.cache_write(wl.new_k, wl.new_v, wl.k_cache, wl.v_cache, wl.slot_mapping,
                       k_scale=wl.k_scale, v_scale=wl.v_scale)
        lens = (wl.context_lens + 1).contiguous()
        out = pa.decode_partitioned(wl.q, wl.k_cache, wl.v_cache, wl.block_table, lens, wl.scale,
                                    wl.partition_size, int(lens.max()), wl.k_scale, wl.v_scale)
    else:
        out = pa.decode_append(wl.q, wl.new_k, wl.new_v, wl.k_cache, wl.v_cache, wl.slot_mapping,
                               wl.block_table, wl.context_lens, wl.scale, k_scale=wl.k_scale,
                               v_scale=wl.v_scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,count", [("worked_example", 0), ("llama7b_mha", 12),
                                        ("gqa", 12), ("fp8_shared_prefix", 12),
                                        ("long_context", 6)])
def test_full_size_step_sampled(name, count):
    print(f"[full-size] {name}", flush=True)
    if count == 0:
        # small enough for the whole oracle, including both caches
        host = workloads.make(name)
        a = oracle_arrays(host)
        ref, kc, vc = oracle.decode_append(
            a["q"], to_numpy_bits(host.new_k), to_numpy_bits(host.new_v), a["k"], a["v"],
            host.slot_mapping.numpy(), a["table"], a["lens"], host.scale, host.num_kv_heads,
            host.block_size, host.q_dtype, host.cache_dtype)
        wl = host.to(DEV)
        out = _step(wl)
        atol, rtol = tol_of(host)
        assert_close(as_f64(out), ref, atol, rtol, name)
        assert to_numpy_bits(wl.k_cache).tobytes() == kc.tobytes()
        assert to_numpy_bits(wl.v_cache).tobytes() == vc.tobytes()
        return
    if name == "long_context":
        wl = workloads.long_context(device=DEV)
    else:
        wl = workloads.make(name).to(DEV)
    pairs = sample_pairs(wl, count)
    captured = capture_step_inputs(wl, pairs)
    out = _step(wl)
    assert torch.isfinite(out).all()
    expect = step_oracle(wl, captured)
    atol, rtol = tol_of(wl)
    got = np.stack([as_f64(out[s, h]) for s, h in pairs])
    assert_close(got, np.stack([e[0] for e in expect]), atol, rtol, f"{name} sampled {pairs}")
    BS = wl.block_size
    for c, (_, k_slot, v_slot) in zip(captured, expect):
        b, o = divmod(c["slot"], BS)
        gk = to_numpy_bits(wl.k_cache[b, c["kvh"], o])
        gv = to_numpy_bits(wl.v_cache[b, c["kvh"], o // 4, :, o % 4])
        assert gk.tobytes() == k_slot.tobytes(), (name, c["s"])
        assert gv.tobytes() == v_slot.tobytes(), (name, c["s"])


def test_full_size_prefill_sampled():
    """The chunked-prefill workload at full size (16 sequences x 512-token
    chunks after up to 1536 cached tokens, Llama-7B shape), in the launch
    configuration bench.py --op prefill times (pa_cache_write, then
    pa_prefill): every output finite; sampled (sequence, head) pairs — all
    512 query rows of each — against the oracle, which writes the chunk into
    host copies of the sequence's own blocks of that kv head taken before
    the step and attends over them."""
    print("[full-size] llama7b_prefill_chunks", flush=True)
    b = workloads.llama7b_prefill_chunks(device=DEV)
    S, H, BS = b.num_seqs, b.num_heads, b.block_size
    G = H // b.num_kv_heads
    cu = b.cu_seqlens_q.cpu().numpy()
    ctx = b.context_lens.cpu().numpy()
    table = b.block_table.cpu().numpy()
    slots = b.slot_mapping.cpu().numpy()
    rng = np.random.default_rng(11)
    seqs = [int(np.argmax(ctx)), int(np.argmin(ctx))] + [int(x) for x in rng.integers(0, S, 3)]
    pairs = [(s, int(rng.integers(0, H))) for s in seqs]
    captured = []
    for s, h in pairs:
        kvh = h // G
        nblk = -(-int(ctx[s]) // BS)
        ids = table[s, :nblk]
        sel = torch.from_numpy(ids.astype(np.int64)).to(DEV)
        rows = slice(int(cu[s]), int(cu[s + 1]))
        # the chunk's slots inside the sequence's own blocks: block j of its table
        pos = {int(p): j for j, p in enumerate(ids)}
        sub = np.array([pos[int(x) // BS] * BS + int(x) % BS for x in slots[rows]], dtype=np.int32)
        captured.append(dict(
            s=s, h=h, nblk=nblk, sub_slots=sub, ctx=int(ctx[s]), n=int(cu[s + 1] - cu[s]),
            q=to_numpy_bits(b.q[rows, h:h + 1]),
            k=to_numpy_bits(b.k_cache.index_select(0, sel)[:, kvh:kvh + 1]),
            v=to_numpy_bits(b.v_cache.index_select(0, sel)[:, kvh:kvh + 1]),
            nk=to_numpy_bits(b.new_k[rows, kvh:kvh + 1]),
            nv=to_numpy_bits(b.new_v[rows, kvh:kvh + 1])))
    pa.cache_write(b.new_k, b.new_v, b.k_cache, b.v_cache, b.slot_mapping)
    out = pa.prefill(b.q, b.k_cache, b.v_cache, b.block_table, b.cu_seqlens_q, b.context_lens,
                     b.scale, b.max_seqlen_q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    atol, rtol = tol_of(b)
    for c in captured:
        k, v = oracle.cache_write(c["nk"], c["nv"], c["k"], c["v"], c["sub_slots"], BS,
                                  b.cache_dtype)
        ref = oracle.paged_prefill(c["q"], k, v, np.arange(c["nblk"], dtype=np.int32)[None, :],
                                   np.array([0, c["n"]], dtype=np.int32),
                                   np.array([c["ctx"]], dtype=np.int32), b.scale, 1, BS,
                                   b.q_dtype, b.cache_dtype)
        got = as_f64(out[int(cu[c["s"]]):int(cu[c["s"] + 1]), c["h"]:c["h"] + 1])
        assert_close(got, ref, atol, rtol, f"prefill sequence {c['s']} head {c['h']}")
