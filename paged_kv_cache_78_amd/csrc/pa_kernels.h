// Internal host-side interface between the C ABI shim and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Dt : int { F16 = 0, BF16 = 1, FP8 = 2 };

// Arguments of the decode kernels (both the one-pass and the partitioned
// form).  Pointers are device pointers; strides are in elements.
struct DecodeParams {
  void* out;                 // [S, H, D] q dtype           (one pass)
  const void* q;             // [S, H, D] row stride q_seq_stride
  const void* k_cache;       // [NB, KVH, BS, D]
  const void* v_cache;       // [NB, KVH, BS/4, D, 4]
  const int32_t* block_table;   // [S, MB]
  const int32_t* context_lens;  // [S]
  float* tmp_out;            // [S, H, NP, D]               (partitioned)
  float* max_logits;         // [S, H, NP]
  float* exp_sums;           // [S, H, NP]
  float qk_scale_log2;       // scale * k_scale * log2(e)
  float v_scale;             // 1 for 16-bit caches
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int64_t q_seq_stride;
  int32_t partition_size;    // tokens per partition (partitioned), else 0
  int32_t num_partitions;    // NP (partitioned), else 1
  int32_t order_by_length;   // one pass: dispatch the longest contexts first
  int32_t die_order;         // vector-ALU partitions: a 1-D grid through die_position
  int32_t num_cus;           // compute units of the device (dispatch order)
  // fused append (one pass only): sequence s's new token k_new/v_new[s]
  // ([KVH, D] rows, token stride kv_token_stride) is stored at
  // slot_mapping[s] (skipped if negative) and attended after the
  // context_lens[s] cached tokens, with the value the cache stores.
  int32_t append;
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int64_t kv_token_stride;
  float k_inv_scale;         // fp32(1/k_scale), fp8 caches
  float v_inv_scale;
};

struct ReduceParams {
  void* out;
  const float* tmp_out;
  const float* max_logits;
  const float* exp_sums;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t partition_size;
  int32_t max_num_partitions;
};

struct CacheWriteParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int64_t num_blocks;
  int64_t kv_token_stride;
  float k_inv_scale;   // fp32(1 / k_scale), fp8 caches only
  float v_inv_scale;
};

// Arguments of the prefill kernel: n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s]
// query tokens of sequence s (packed rows of q and out) attend the
// context_lens[s] cached tokens, the queries being the last n_s positions.
struct PrefillParams {
  void* out;                    // [total_q, H, D] q dtype, contiguous
  const void* q;                // [total_q, H, D] row stride q_token_stride
  const void* k_cache;          // [NB, KVH, BS, D]
  const void* v_cache;          // [NB, KVH, BS/4, D, 4]
  const int32_t* block_table;   // [S, MB]
  const int32_t* cu_seqlens_q;  // [S + 1]
  const int32_t* context_lens;  // [S]
  float qk_scale_log2;          // scale * k_scale * log2(e)
  float v_scale;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int64_t q_token_stride;
  int32_t total_q;
  int32_t max_seqlen_q;         // bounds every n_s (grid size)
  int32_t causal;
};

// Whole-block copy between two pools (one may live in pinned host memory,
// given by its device-side address).  mapping [num_pairs, 2] = (src, dst)
// block ids; pairs with an id out of range are skipped.
struct BlockCopyParams {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* mapping;
  int32_t num_pairs;
  int64_t src_num_blocks;
  int64_t dst_num_blocks;
  int64_t block_bytes;   // bytes of one block of K (= of V), a multiple of 16
};

// Each returns hipSuccess or the launch error.  Shapes are validated by the
// caller; the launchers only pick the instantiation.
hipError_t launch_decode_valu(const DecodeParams& p, Dt q_dt, Dt cache_dt, int head_size,
                              int block_size, bool partitioned, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, Dt q_dt, Dt cache_dt, int head_size,
                              int block_size, bool partitioned, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, Dt out_dt, int head_size, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteParams& p, Dt in_dt, Dt cache_dt, int head_size,
                              int block_size, hipStream_t stream);
hipError_t launch_copy_blocks(const BlockCopyParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, Dt q_dt, Dt cache_dt, int head_size,
                          int block_size, hipStream_t stream);

}  // namespace pa
