"""One small parity case for every compiled decode kernel, through the C ABI:
the vector-ALU kernel (one query head per kv head) and the matrix-core
kernel (grouped heads), each for f16 and bf16 queries over 16-bit and fp8
e4m3fn caches, head sizes 64 and 128, block sizes 16 and 32, run in one pass
(pa_decode), split into partitions merged by pa_reduce
(pa_decode_partitioned), and as the fused step that stores the new token
first (pa_decode_append).  Every slot outside the contexts holds NaN."""
import pytest
import torch

import oracle
import paged_kv_cache_78_amd as pa
import workloads
from gpu_helpers import as_f64, assert_close, oracle_arrays, oracle_decode, tol_of
from workloads import to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _workload(qd, cache, D, BS, G):
    H, KVH = 2 * G, 2
    if cache == "e4m3fn":
        wl = workloads.fp8_shared_prefix(seed=61, num_seqs=8, median=150.0, cap=400, num_heads=H,
                                         num_kv_heads=KVH, head_size=D, block_size=BS,
                                         prefix_tokens=2 * BS)
        if qd == "f16":
            # the bf16 queries and new tokens (N(0,1)) are exact in f16
            wl = workloads.synth.replace(wl, q=wl.q.to(torch.float16),
                                         new_k=wl.new_k.to(torch.float16),
                                         new_v=wl.new_v.to(torch.float16), q_dtype="f16")
    else:
        wl = workloads.gqa(seed=62, num_seqs=7, len_range=(1, 300), num_heads=H, num_kv_heads=KVH,
                           head_size=D, block_size=BS, dtype=qd,
                           lengths=[1, BS - 1, BS + 1, 5 * BS + 3, 257])
    assert wl.q_dtype == qd and wl.cache_dtype == cache
    return workloads.poison_unused_slots(wl)


@pytest.mark.parametrize("mode", ["one_pass", "partitioned", "append"])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("BS", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("qd,cache", [("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3fn"),
                                      ("bf16", "e4m3fn")])
def test_every_decode_kernel(qd, cache, D, BS, G, mode):
    what = f"{qd}/{cache} D{D} BS{BS} G{G} {mode}"
    print(f"[decode sweep] {what}", flush=True)
    wl = _workload(qd, cache, D, BS, G)
    g = wl.to(DEV)
    atol, rtol = tol_of(wl)
    if mode == "one_pass":
        out = pa.decode(g.q, g.k_cache, g.v_cache, g.block_table, g.context_lens, wl.scale,
                        k_scale=wl.k_scale, v_scale=wl.v_scale)
        torch.cuda.synchronize()
        assert_close(as_f64(out), oracle_decode(wl), atol, rtol, what)
    elif mode == "partitioned":
        # partitions of 2 blocks: several per sequence, and a ragged last one
        maxL = int(wl.context_lens.max())
        out = pa.decode_partitioned(g.q, g.k_cache, g.v_cache, g.block_table, g.context_lens,
                                    wl.scale, 2 * BS, maxL, wl.k_scale, wl.v_scale)
        torch.cuda.synchronize()
        assert_close(as_f64(out), oracle_decode(wl), atol, rtol, what)
    else:
        out = pa.decode_append(g.q, g.new_k, g.new_v, g.k_cache, g.v_cache, g.slot_mapping,
                               g.block_table, g.context_lens, wl.scale, k_scale=wl.k_scale,
                               v_scale=wl.v_scale)
        torch.cuda.synchronize()
        a = oracle_arrays(wl)
        ref, kc, vc = oracle.decode_append(a["q"], to_numpy_bits(wl.new_k),
                                           to_numpy_bits(wl.new_v), a["k"], a["v"],
                                           wl.slot_mapping.cpu().numpy(), a["table"], a["lens"],
                                           wl.scale, wl.num_kv_heads, wl.block_size, wl.q_dtype,
                                           wl.cache_dtype, wl.k_scale, wl.v_scale)
        assert_close(as_f64(out), ref, atol, rtol, what)
        assert to_numpy_bits(g.k_cache).tobytes() == kc.tobytes(), what
        assert to_numpy_bits(g.v_cache).tobytes() == vc.tobytes(), what


@pytest.mark.parametrize("mode", ["one_pass", "partitioned", "append"])
def test_vector_alu_plain_grid(mode):
    """The vector-ALU kernel's launches beyond the die order's item limit (a
    3-D partition grid; one pass in index order), reached through the library
    built with that limit at zero: the same parity as the default build."""
    import os
    import paged_kv_cache_78_amd.binding as B
    path = os.path.join(os.path.dirname(B.__file__), "variants", "libpa_plain_grid.so")
    what = f"plain grid {mode}"
    print(f"[decode sweep] {what}", flush=True)
    saved_path, saved_lib = B._LIB_PATH, B._lib
    try:
        B._LIB_PATH, B._lib = path, None
        for qd in ("f16", "bf16"):
            wl = _workload(qd, qd, 128, 16, 1)
            g = wl.to(DEV)
            atol, rtol = tol_of(wl)
            if mode == "one_pass":
                out = pa.decode(g.q, g.k_cache, g.v_cache, g.block_table, g.context_lens, wl.scale)
                torch.cuda.synchronize()
                assert_close(as_f64(out), oracle_decode(wl), atol, rtol, what)
            elif mode == "partitioned":
                out = pa.decode_partitioned(g.q, g.k_cache, g.v_cache, g.block_table,
                                            g.context_lens, wl.scale, 32, int(wl.context_lens.max()))
                torch.cuda.synchronize()
                assert_close(as_f64(out), oracle_decode(wl), atol, rtol, what)
            else:
                out = pa.decode_append(g.q, g.new_k, g.new_v, g.k_cache, g.v_cache, g.slot_mapping,
                                       g.block_table, g.context_lens, wl.scale)
                torch.cuda.synchronize()
                a = oracle_arrays(wl)
                ref, kc, vc = oracle.decode_append(a["q"], to_numpy_bits(wl.new_k),
                                                   to_numpy_bits(wl.new_v), a["k"], a["v"],
                                                   wl.slot_mapping.cpu().numpy(), a["table"],
                                                   a["lens"], wl.scale, wl.num_kv_heads,
                                                   wl.block_size, wl.q_dtype, wl.cache_dtype)
                assert_close(as_f64(out), ref, atol, rtol, what)
                assert to_numpy_bits(g.k_cache).tobytes() == kc.tobytes(), what
                assert to_numpy_bits(g.v_cache).tobytes() == vc.tobytes(), what
    finally:
        B._LIB_PATH, B._lib = saved_path, saved_lib
