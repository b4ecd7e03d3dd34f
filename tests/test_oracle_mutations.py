"""The oracle's pins catch plausible mistakes: each case plants one mistake in
the oracle (on the CPU, through monkeypatch) and checks that at least one of
the pin tests then fails."""
import numpy as np
import pytest

import oracle
import oracle.formats as fmt
import oracle.paged_attention as pa_oracle
import test_oracle_attention as t_att
import test_oracle_cache_write as t_cw
import test_oracle_fp8 as t_fp8
import test_oracle_indexing as t_idx

ATTENTION_PINS = [
    lambda: t_att.test_brute_force_tiny(0),
    lambda: t_att.test_sdpa_library_case(8, 2),
    lambda: t_att.test_bf16_and_fp8_inputs_match_sdpa_on_dequantised_values(),
    lambda: t_att.test_two_tokens_closed_form(),
    lambda: t_att.test_partition_merge_equals_unpartitioned(16),
    lambda: t_att.test_partition_triples_against_brute_force(),
]


def _fails(pins) -> bool:
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def test_unmutated_oracle_passes_every_pin():
    assert not _fails(ATTENTION_PINS)


def test_dropped_scale_is_caught(monkeypatch):
    orig = pa_oracle.decode_sequence

    def no_scale(q_s, k_cache, v_cache, table_row, context_len, scale, *a, **kw):
        return orig(q_s, k_cache, v_cache, table_row, context_len, 1.0, *a, **kw)
    monkeypatch.setattr(pa_oracle, "decode_sequence", no_scale)
    assert _fails(ATTENTION_PINS)


def test_wrong_kv_head_mapping_is_caught(monkeypatch):
    def interleaved(q_s, k_cache, v_cache, table_row, context_len, scale, num_kv_heads,
                    block_size, cache_fmt, k_scale=1.0, v_scale=1.0, heads=None,
                    return_probs=False):
        # query head h reads kv head h % KVH instead of h // G
        H, D = q_s.shape
        heads = list(range(H)) if heads is None else list(heads)
        L = int(context_len)
        n = oracle.num_logical_blocks(L, block_size)
        ids = np.asarray(table_row[:n], dtype=np.int64)
        out = np.zeros((len(heads), D))
        for i, h in enumerate(heads):
            if L == 0:
                continue
            kvh = h % num_kv_heads
            K = oracle.to_f64(k_cache[ids, kvh], cache_fmt).reshape(n * block_size, D)[:L]
            V = oracle.v_tiles_to_rows(oracle.to_f64(v_cache[ids, kvh], cache_fmt))[:L]
            x = np.float64(np.float32(scale)) * (K @ q_s[h])
            _, _, p = oracle.softmax_stats(x)
            out[i] = p @ V
        return out
    monkeypatch.setattr(pa_oracle, "decode_sequence", interleaved)
    assert _fails([lambda: t_att.test_sdpa_library_case(8, 2)])


def test_transposed_v_quad_is_caught(monkeypatch):
    def bad_rows(vt):
        n, q4, D, four = vt.shape
        return vt.reshape(n * q4 * four, D)          # forgets the [quad, dim, token] order
    monkeypatch.setattr(pa_oracle, "v_tiles_to_rows", bad_rows)
    assert _fails(ATTENTION_PINS)


def test_off_by_one_slot_is_caught(monkeypatch):
    def bad_slots(row, L, bs):
        return [(int(row[(t + 1) // bs]), (t + 1) % bs) for t in range(int(L))]
    monkeypatch.setattr(pa_oracle, "token_slots", bad_slots)
    monkeypatch.setattr(oracle, "token_slots", bad_slots)
    assert _fails([t_idx.test_block_table_example_blocks_read, t_idx.test_decode_walkthrough_example])


def test_merge_without_rescale_is_caught(monkeypatch):
    def bad_merge(partials):
        if not partials:
            return None
        w = [l for _, l, _ in partials]              # drops e^(m_p - M)
        return sum((wi / sum(w)) * o for wi, (_, _, o) in zip(w, partials))
    monkeypatch.setattr(pa_oracle, "merge_partials", bad_merge)
    assert _fails([lambda: t_att.test_partition_merge_equals_unpartitioned(16)])


def test_wrong_fp8_bias_is_caught(monkeypatch):
    def bad_decode(codes):
        c = codes.astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(np.float64)
        mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 8.0))
        return sign * mag
    monkeypatch.setattr(fmt, "e4m3fn_to_f64", bad_decode)
    monkeypatch.setattr(oracle, "e4m3fn_to_f64", bad_decode)
    assert _fails([t_fp8.test_decode_spot_values_from_the_definition,
                   t_fp8.test_decode_matches_torch_on_every_code])


def test_fp8_round_half_up_is_caught(monkeypatch):
    import math

    def bad_round(y):
        if y != y:
            return y
        y = max(-448.0, min(448.0, y))
        a = abs(y)
        e = max(math.floor(math.log2(a)), -6) if a > 0 else -6
        q = 2.0 ** (e - 3)
        return math.copysign(math.floor(a / q + 0.5) * q, y)   # ties away from zero
    monkeypatch.setattr(fmt, "e4m3fn_round", bad_round)
    assert _fails([t_fp8.test_encode_all_fp16_inputs_brute_force_nearest])


def test_cache_write_wrong_v_position_is_caught(monkeypatch):
    def bad_write(k, v, k_cache, v_cache, slot_mapping, block_size, cache_fmt, k_scale=1.0,
                  v_scale=1.0):
        kc, vc = k_cache.copy(), v_cache.copy()
        for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
            if slot < 0:
                continue
            b, o = divmod(int(slot), block_size)
            kc[b, :, o, :] = k[i]
            vc[b, :, o % 4, :, o // 4 % 4] = v[i]   # quad and lane swapped
        return kc, vc
    monkeypatch.setattr(pa_oracle, "cache_write", bad_write)
    monkeypatch.setattr(oracle, "cache_write", bad_write)
    assert _fails([t_cw.test_write_then_decode_attends_the_new_token])


def test_append_without_quantising_the_new_token_is_caught(monkeypatch):
    import test_oracle_decode_append as t_app

    def raw_rows(x, cache_fmt, scale=1.0):
        return oracle.to_f64(x, pa_oracle._fmt_of(x))      # skips the fp8 round trip
    monkeypatch.setattr(pa_oracle, "stored_rows", raw_rows)
    assert _fails([lambda: t_app.test_equals_write_then_decode_one_longer("e4m3fn"),
                   t_app.test_empty_context_gives_the_new_value])


def test_append_that_drops_the_new_token_is_caught(monkeypatch):
    import test_oracle_decode_append as t_app
    orig = pa_oracle.stored_rows

    def tiny_rows(x, cache_fmt, scale=1.0):
        return orig(x, cache_fmt, scale) * 0.0               # new token contributes a zero row
    monkeypatch.setattr(pa_oracle, "stored_rows", tiny_rows)
    assert _fails([t_app.test_worked_example_by_hand])


def test_copy_that_forgets_v_is_caught(monkeypatch):
    import oracle.block_ops as bo
    import test_oracle_block_ops as t_blk

    def k_only(src_k, src_v, dst_k, dst_v, mapping):
        out_k, out_v = np.array(dst_k, copy=True), np.array(dst_v, copy=True)
        for s, d in np.asarray(mapping).reshape(-1, 2).tolist():
            if 0 <= s < src_k.shape[0] and 0 <= d < out_k.shape[0]:
                out_k[d] = src_k[s]
        return out_k, out_v
    monkeypatch.setattr(bo, "copy_blocks", k_only)
    monkeypatch.setattr(oracle, "copy_blocks", k_only)
    assert _fails([t_blk.test_copy_by_hand, t_blk.test_swap_out_and_back_in_restores_the_attention])


def test_cow_without_repointing_is_caught(monkeypatch):
    import oracle.block_ops as bo
    import test_oracle_block_ops as t_blk
    orig = bo.cow_step

    def no_repoint(table_row, context_len, block_size, ref_counts, free_list):
        pair, _ = orig(table_row, context_len, block_size, ref_counts, free_list)
        return pair, list(table_row)                 # copies but keeps writing the shared block
    monkeypatch.setattr(bo, "cow_step", no_repoint)
    monkeypatch.setattr(oracle, "cow_step", no_repoint)
    assert _fails([t_blk.test_cow_then_write_keeps_the_other_sequence_and_gives_the_writer_its_token])


def _prefill_variant(last_of):
    """paged_prefill with another rule for the last key a query attends."""
    def run(q, k_cache, v_cache, block_table, cu_seqlens_q, context_lens, scale, num_kv_heads,
            block_size, q_fmt, cache_fmt, k_scale=1.0, v_scale=1.0, causal=True, seqs=None):
        T, H, D = q.shape
        cu = [int(x) for x in cu_seqlens_q]
        G = H // num_kv_heads
        out = np.zeros((T, H, D))
        for s in range(len(cu) - 1):
            Ks, n = int(context_lens[s]), cu[s + 1] - cu[s]
            ids = np.asarray(block_table[s, :oracle.num_logical_blocks(Ks, block_size)],
                             dtype=np.int64)
            for i in range(n):
                last = last_of(Ks, n, i) if causal else Ks - 1
                if last < 0:
                    continue
                for h in range(H):
                    K = oracle.to_f64(k_cache[ids, h // G], cache_fmt).reshape(-1, D)[:last + 1]
                    V = oracle.v_tiles_to_rows(oracle.to_f64(v_cache[ids, h // G],
                                                             cache_fmt))[:last + 1]
                    x = np.float64(np.float32(scale)) * (K @ oracle.to_f64(q[cu[s] + i, h], q_fmt))
                    _, _, p = oracle.softmax_stats(x)
                    out[cu[s] + i, h] = p @ V
        return out
    return run


def test_prefill_top_left_alignment_is_caught(monkeypatch):
    import test_oracle_prefill as t_pf
    bad = _prefill_variant(lambda Ks, n, i: min(i, Ks - 1))
    monkeypatch.setattr(pa_oracle, "paged_prefill", bad)
    monkeypatch.setattr(oracle, "paged_prefill", bad)
    assert _fails([t_pf.test_two_chunks_equal_one, t_pf.test_example_shapes_with_causal_alignment])


def test_prefill_off_by_one_mask_is_caught(monkeypatch):
    import test_oracle_prefill as t_pf
    bad = _prefill_variant(lambda Ks, n, i: Ks - n + i - 1)
    monkeypatch.setattr(pa_oracle, "paged_prefill", bad)
    monkeypatch.setattr(oracle, "paged_prefill", bad)
    assert _fails([t_pf.test_brute_force_tiny, lambda: t_pf.test_sdpa_with_explicit_mask(True)])


def test_block_manager_lifo_free_list_is_caught(monkeypatch):
    import oracle.block_manager as bmod
    import test_oracle_block_manager as t_bm

    def release_front(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            self.free.insert(0, b)                   # freed blocks reused first
    monkeypatch.setattr(bmod._Pool, "release", release_front)
    assert _fails([t_bm.test_allocation_from_the_front_and_release_to_the_back,
                   t_bm.test_swap_out_and_in])


def test_block_manager_without_copy_on_write_is_caught(monkeypatch):
    import oracle.block_manager as bmod
    import test_oracle_block_manager as t_bm

    def append_in_place(self, sid):
        st = self.seqs[sid]
        pos = st["len"]
        j = pos // self.bs
        if j == len(st["blocks"]):
            st["blocks"].append(self.gpu.take(1)[0])
        st["len"] = pos + 1
        return st["blocks"][j] * self.bs + pos % self.bs, None
    monkeypatch.setattr(bmod.BlockManager, "append_slot", append_in_place)
    assert _fails([t_bm.test_fork_shares_and_copy_on_write_splits])


FP8_QUANTISER_PINS = [t_fp8.test_quantiser_takes_the_binary32_reciprocal_and_a_binary32_product,
                      t_fp8.test_cache_write_fp8_code_of_a_bf16_value_at_a_rounding_boundary]


def _patch_quantiser(monkeypatch, fn):
    monkeypatch.setattr(fmt, "quantise_e4m3fn", fn)
    monkeypatch.setattr(oracle, "quantise_e4m3fn", fn)
    monkeypatch.setattr(pa_oracle, "quantise_e4m3fn", fn)


def test_unmutated_quantiser_passes_its_pins():
    assert not _fails(FP8_QUANTISER_PINS)


def test_fp8_quantiser_that_divides_by_the_scale_is_caught(monkeypatch):
    def divides(x, scale):
        y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
        return fmt.e4m3fn_encode(y, np.float32(1.0))
    _patch_quantiser(monkeypatch, divides)
    for pin in FP8_QUANTISER_PINS:
        assert _fails([pin])


def test_fp8_quantiser_with_fp64_reciprocal_and_product_is_caught(monkeypatch):
    def fp64_product(x, scale):
        y = np.asarray(x, dtype=np.float32).astype(np.float64) * (1.0 / float(np.float32(scale)))
        flat = [fmt._e4m3fn_code_of_value(fmt.e4m3fn_round(float(t))) for t in y.reshape(-1)]
        return np.array(flat, dtype=np.uint8).reshape(y.shape)
    _patch_quantiser(monkeypatch, fp64_product)
    for pin in FP8_QUANTISER_PINS:
        assert _fails([pin])
