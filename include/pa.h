/*
 * pa.h — C ABI of the paged decode-attention library (libpa.so, HIP for gfx950).
 *
 * What the library computes (cited by page and section):
 *   - Paged KV cache: K/V vectors live in fixed-size blocks of `block_size`
 *     tokens scattered through a physical pool; a per-sequence block table maps
 *     logical block j (tokens j*block_size .. j*block_size+block_size-1) to a
 *     physical block; -1 marks an unallocated entry.
 *     ("How does paged attention work (in detail)", sections 2 and 4.1;
 *      "Paged attention" wiki, decode path and its example.)
 *   - Decode attention: one query token per sequence attends, for every head,
 *     over the sequence's whole context: x_t = scale * <q, k_t>, softmax
 *     m = max x, f = exp(x - m), l = sum f, p = f / l, out = sum p_t v_t.
 *     (vLLM "Paged Attention" design page, sections "QK", "Softmax", "Value",
 *      "LV" and "Output".)
 *   - Cache write: a new token's K/V goes to its slot inside a physical block.
 *     ("How does paged attention work", section 4.1 step 5; vLLM paper summary,
 *      section 3 "Decoding".)
 *   - Split-context partitions whose partial results are merged
 *     (the design page's max_num_partitions grid dimension and per-partition
 *      output slot, section "Output"); the merge rule is derived from the
 *      softmax definition.
 *
 * Layouts (row-major, element type `cache_dtype`):
 *   k_cache [num_blocks, num_kv_heads, block_size, head_size]   token-major tile
 *   v_cache [num_blocks, num_kv_heads, block_size/4, head_size, 4]
 *           quad-interleaved tile: token t of a block, head dim d, sits at
 *           [t / 4, d, t % 4] (four consecutive tokens of one dim are
 *           adjacent, the dims of one token quad follow each other)
 *   q       [num_seqs, num_heads, head_size] with row stride q_seq_stride
 *   out     [num_seqs, num_heads, head_size] contiguous, element type q_dtype
 *   block_table  [num_seqs, max_blocks_per_seq] int32
 *   context_lens [num_seqs] int32: tokens attended by sequence s (positions
 *                0 .. context_lens[s]-1).  A decode step writes the new token
 *                at position L with pa_cache_write, then decodes with L + 1,
 *                or does both in one launch with pa_decode_append.
 * Query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Element types: q/out f16 or bf16; caches f16, bf16 (same type as q) or
 * fp8 e4m3fn (OCP) with one fp32 scale per cache: value = code * k_scale
 * (resp. v_scale).  Scales are ignored for 16-bit caches.
 *
 * Alignment: q, out, k, v, the caches and tmp_out start on 16-byte
 * boundaries and q_seq_stride / kv_token_stride are multiples of 8 elements
 * (rows move as 16-byte pieces); anything else gives PA_ERR_SHAPE.
 *
 * Ownership and execution: every array pointer is a device pointer
 * (pa_copy_blocks also takes pinned host memory) owned by the caller; inputs are only read; only out, the caches (pa_cache_write,
 * pa_decode_append, pa_copy_blocks) and
 * the workspace arrays are written.  The library allocates nothing and keeps
 * no state, apart from the static scratch array of
 * pa_decode_partitioned_noalloc.  All calls are asynchronous on `stream` (a hipStream_t; NULL is
 * the default stream); a PA_OK return means "launched", not "finished".
 *
 * Errors: arguments the host can check are checked before any launch and give
 * a negative pa_status with nothing launched.  Errors only visible in device
 * data (a block id outside [0, num_blocks) inside a context, a context longer
 * than the table or than max_context_len, a negative context length) are not
 * reported: the affected (sequence, head) output row is written as NaN and no
 * address derived from the bad entry is read.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F16 = 0,
  PA_BF16 = 1,
  PA_FP8_E4M3FN = 2,
  /* Range markers, never valid element types: they make every int32 value a
   * value of pa_dtype, so that a call passing an unknown type is rejected
   * with PA_ERR_DTYPE rather than reading an out-of-range enum (undefined
   * in C++).  The type stays int-sized. */
  PA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PA_DTYPE_RANGE_MAX_ = 2147483647
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  PA_ERR_SHAPE = -2,       /* a size is <= 0 or sizes are inconsistent      */
  PA_ERR_UNSUPPORTED = -3, /* head size / block size / group not built      */
  PA_ERR_DTYPE = -4,       /* element type combination not supported        */
  PA_ERR_WORKSPACE = -5,   /* partition size or workspace invalid           */
  PA_ERR_HIP = -6,         /* the HIP runtime refused the launch            */
  PA_ERR_MEMORY = -7,      /* a pool is not device-accessible memory        */
  PA_ERR_NO_BLOCKS = -8,   /* block manager: not enough free blocks         */
  PA_ERR_SEQUENCE = -9,    /* block manager: unknown, duplicate or swapped-
                              out sequence for this call                    */
  PA_ERR_SCRATCH = -10     /* pa_decode_partitioned_noalloc: the partials do
                              not fit in the library's static scratch       */
} pa_status;

/* Static text for a status code (never NULL). */
const char* pa_status_string(int status);

/* Version of this ABI (incremented on any signature or layout change). */
int pa_abi_version(void);

/*
 * pa_cache_write — store num_tokens new K/V vectors into their cache slots.
 *   k, v          [num_tokens, num_kv_heads, head_size] (row stride
 *                 kv_token_stride elements; heads contiguous), in_dtype.
 *   slot_mapping  [num_tokens] int32: slot = physical_block * block_size +
 *                 offset; a negative slot skips the token.
 *   Writes k[i, h, :] to k_cache[slot / BS, h, slot % BS, :] and v[i, h, :]
 *   to v_cache[slot / BS, h, (slot % BS) / 4, :, slot % 4]; nothing else is
 *   written.
 *   16-bit caches: cache_dtype == in_dtype, bits copied unchanged.
 *   fp8 cache: code = e4m3fn(clamp(x * (1/scale), -448, 448)) rounded to
 *   nearest even, with 1/scale computed once in fp32 on the host and the
 *   product taken in fp32; NaN stays NaN.
 *   Slots >= num_blocks * block_size are skipped (caller error); two tokens
 *   with the same slot is a caller error (which one wins is unspecified).
 * Supported: head_size in {64, 128}, block_size in {16, 32}.
 */
int pa_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                   const int32_t* slot_mapping, int32_t num_tokens,
                   int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                   int64_t num_blocks, int64_t kv_token_stride,
                   pa_dtype in_dtype, pa_dtype cache_dtype,
                   float k_scale, float v_scale, void* stream);

/*
 * pa_decode — decode attention over the paged cache in one pass.
 *   out[s, h, :] = sum_t p_t * V_s[t, h / G, :] with p the softmax of
 *   scale * <q[s, h, :], K_s[t, h / G, :]> over t < context_lens[s]
 *   (G = num_heads / num_kv_heads); context_lens[s] == 0 gives zeros.
 *   Entries of block_table past ceil(context_lens[s] / block_size) are never
 *   read (they may be -1).  Deterministic: the same inputs give the same bits.
 * Supported: head_size in {64, 128}; block_size in {16, 32}; G in [1, 16];
 *   q_dtype in {f16, bf16}; cache_dtype == q_dtype or PA_FP8_E4M3FN.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens,
              float scale, int32_t num_kv_heads, int32_t block_size,
              int32_t num_seqs, int32_t num_heads, int32_t head_size,
              int32_t max_blocks_per_seq, int64_t num_blocks, int64_t q_seq_stride,
              pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale, float v_scale,
              void* stream);

/*
 * pa_decode_append — one decode step in one launch: store each sequence's
 * new token and attend over its cached context plus that token.
 *   k, v          [num_seqs, num_kv_heads, head_size] (row stride
 *                 kv_token_stride elements), q_dtype: the new token of each
 *                 sequence.
 *   slot_mapping  [num_seqs] int32: the new token's slot (as in
 *                 pa_cache_write; negative: not stored).
 *   Stores k[s], v[s] exactly as pa_cache_write does, and writes
 *   out[s, h, :] = attention of q[s, h, :] over positions
 *   0 .. context_lens[s] - 1 of the cache (read through block_table) and
 *   the new token, whose K/V enter with the values the cache stores for
 *   them (fp8: quantised).  When slot_mapping[s] is the slot of position
 *   context_lens[s] this equals pa_cache_write followed by pa_decode with
 *   context_lens[s] + 1 (the cache-write and decode steps of the decode
 *   phase, "How does paged attention work (in detail)", section 4.1, and the
 *   vLLM paper summary, section 3 "Decoding").
 *   The new token is taken from k/v, never read back from the cache.  A slot
 *   that some sequence of the same call reads inside its context is a caller
 *   error (the read races with the store).  Bad device data as in pa_decode:
 *   the row is NaN; the token is still stored.
 * Same support matrix as pa_decode (one pass only).
 */
int pa_decode_append(void* out, const void* q, const void* k, const void* v,
                     void* k_cache, void* v_cache, const int32_t* slot_mapping,
                     const int32_t* block_table, const int32_t* context_lens,
                     float scale, int32_t num_kv_heads, int32_t block_size,
                     int32_t num_seqs, int32_t num_heads, int32_t head_size,
                     int32_t max_blocks_per_seq, int64_t num_blocks, int64_t q_seq_stride,
                     int64_t kv_token_stride, pa_dtype q_dtype, pa_dtype cache_dtype,
                     float k_scale, float v_scale, void* stream);

/*
 * pa_prefill — varlen / chunked prefill attention over the paged cache.
 *   q             [total_q, num_heads, head_size] (row stride q_token_stride
 *                 elements), the query tokens of all sequences packed:
 *                 sequence s owns rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
 *                 ("Paged attention" wiki, Varlen path: cu_seq_lens).
 *   cu_seqlens_q  [num_seqs + 1] int32, cu_seqlens_q[0] = 0, non-decreasing.
 *   context_lens  [num_seqs] int32: K_s tokens of sequence s in the cache
 *                 (read through block_table), including the chunk's own
 *                 tokens, which the caller wrote first (pa_cache_write).
 *   With n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s], query i of sequence s is
 *   position K_s - n_s + i (the chunk is the sequence's last n_s tokens) and
 *   out[cu_seqlens_q[s] + i, h, :] is its attention over keys
 *   0 .. K_s - n_s + i (causal != 0) or over all K_s keys (causal == 0); a
 *   query with no key gives zeros.  out [total_q, num_heads, head_size],
 *   q_dtype, contiguous.
 *   max_seqlen_q must bound every n_s (it sizes the grid): a larger n_s, a
 *   bad block id in the keys read or K_s outside [0, max_blocks_per_seq *
 *   block_size] gives NaN rows; rows of a sequence whose cu_seqlens_q range
 *   is empty, decreasing or outside [0, total_q] are not written.
 * Same support matrix as pa_decode (G = num_heads / num_kv_heads in [1, 16]).
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* cu_seqlens_q,
               const int32_t* context_lens, float scale, int32_t num_kv_heads,
               int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t head_size,
               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t total_q,
               int32_t max_seqlen_q, int64_t q_token_stride, int32_t causal,
               pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale, float v_scale,
               void* stream);

/*
 * pa_copy_blocks — copy whole physical blocks (K and V, every kv head) from
 * one pool to another, or inside one pool.
 *   src_k/src_v   [src_num_blocks, num_kv_heads, ...] one block = one
 *                 contiguous run of num_kv_heads * block_size * head_size
 *                 elements of cache_dtype in each of K and V (both cache
 *                 layouts above).
 *   dst_k/dst_v   [dst_num_blocks, ...] likewise.
 *   block_mapping [num_pairs, 2] int32 (src block, dst block); a pair with a
 *                 negative or out-of-range id is skipped.
 *   Uses: copy-on-write of a shared block before a sequence writes into it
 *   (src pool == dst pool; "How does paged attention work (in detail)",
 *   section 3.3), and swapping a preempted sequence's blocks out to a CPU
 *   pool and back (same page, section 4.3; vLLM paper summary, section 5).
 *   Pools and block_mapping may be device memory or pinned host memory
 *   (hipHostMalloc; the kernel reads and writes it over the host link);
 *   pageable host memory gives PA_ERR_MEMORY.  Bytes are copied unchanged.
 *   A dst block listed twice, or a block that is both a source and a
 *   destination of the same call, is a caller error (unspecified result).
 *   num_pairs <= 65535.  Supported: head_size in {64, 128}, block_size in
 *   {16, 32}.
 */
int pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* block_mapping, int32_t num_pairs,
                   int64_t src_num_blocks, int64_t dst_num_blocks,
                   int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                   pa_dtype cache_dtype, void* stream);

/*
 * Workspace of pa_decode_partitioned, in bytes, for
 * NP = ceil(max_context_len / partition_size) partitions:
 *   tmp_out    [num_seqs, num_heads, NP, head_size] fp32
 *   max_logits [num_seqs, num_heads, NP] fp32
 *   exp_sums   [num_seqs, num_heads, NP] fp32
 * (three separate arrays; this returns their total).  0 on invalid sizes.
 */
size_t pa_partition_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                    int32_t head_size, int32_t max_context_len,
                                    int32_t partition_size);

/*
 * pa_decode_partitioned — split each context into partitions of
 * partition_size tokens (a multiple of block_size) and write, for partition
 * p < ceil(context_lens[s] / partition_size):
 *   max_logits[s, h, p] = m_p = max of scale * <q, k_t> over the partition
 *   exp_sums[s, h, p]   = l_p = sum_t exp(x_t - m_p)
 *   tmp_out[s, h, p, :] = o_p = sum_t exp(x_t - m_p) v_t / l_p
 * Partitions p >= that count are not written.  max_context_len bounds every
 * context_lens[s] (a longer context gives a NaN row in pa_reduce) and sets
 * the partition count NP = ceil(max_context_len / partition_size).
 * Same support matrix as pa_decode.
 */
int pa_decode_partitioned(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* context_lens,
                          float scale, int32_t num_kv_heads, int32_t block_size,
                          int32_t num_seqs, int32_t num_heads, int32_t head_size,
                          int32_t max_blocks_per_seq, int64_t num_blocks,
                          int64_t q_seq_stride, pa_dtype q_dtype, pa_dtype cache_dtype,
                          float k_scale, float v_scale, int32_t partition_size,
                          int32_t max_context_len, float* tmp_out, float* max_logits,
                          float* exp_sums, void* stream);

/*
 * pa_reduce — merge the partitions written by pa_decode_partitioned:
 *   M = max_p m_p, l = sum_p l_p exp(m_p - M),
 *   out[s, h, :] = sum_p (l_p exp(m_p - M) / l) o_p      (p < NP_s)
 * with NP_s = ceil(context_lens[s] / partition_size); context 0 gives zeros;
 * NP_s > max_num_partitions or a NaN partial gives a NaN row.
 *   out [num_seqs, num_heads, head_size] out_dtype (f16 or bf16).
 *   max_num_partitions <= 15360 (one fp32 weight per partition is staged in
 *   LDS); larger gives PA_ERR_WORKSPACE.
 */
int pa_reduce(void* out, const float* tmp_out, const float* max_logits,
              const float* exp_sums, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t head_size, int32_t partition_size,
              int32_t max_num_partitions, pa_dtype out_dtype, void* stream);

/*
 * pa_decode_partitioned_noalloc — for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): pa_decode_partitioned followed by pa_reduce into out,
 * with the partial triples kept in a static device array of the library
 * (PA_NOALLOC_SCRATCH_BYTES per GPU, created when the library is loaded on
 * that GPU and held until the process ends) instead of a caller workspace.
 *   Arguments and result as pa_decode_partitioned + pa_reduce (out
 *   [num_seqs, num_heads, head_size], q_dtype).  Calls no hipMalloc/hipFree.
 *   The partials need S * H * NP * head_size * 4 bytes plus 2 * S * H * NP * 4
 *   (NP = ceil(max_context_len / partition_size); each array rounded up to
 *   256 bytes); more than PA_NOALLOC_SCRATCH_BYTES gives PA_ERR_SCRATCH and
 *   nothing is launched, as does NP > 15360 (PA_ERR_WORKSPACE).
 *   Every call on one GPU uses the same array: calls that overlap on one GPU
 *   (different streams, or host threads) race and give wrong results; calls
 *   ordered on one stream are safe.  Nothing in the array needs clearing:
 *   the merge reads only partitions the same call wrote.
 */
#define PA_NOALLOC_SCRATCH_BYTES (48u << 20)
int pa_decode_partitioned_noalloc(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* context_lens, float scale,
                                  int32_t num_kv_heads, int32_t block_size, int32_t num_seqs,
                                  int32_t num_heads, int32_t head_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int64_t q_seq_stride, pa_dtype q_dtype, pa_dtype cache_dtype,
                                  float k_scale, float v_scale, int32_t partition_size,
                                  int32_t max_context_len, void* stream);

/*
 * Host block manager (CPU code; no GPU call, no stream).  It decides where
 * every token's K/V lives: the block tables, slot_mapping and block copies
 * the kernels above consume.  "How does paged attention work (in detail)",
 * sections 2-4: free blocks wait in a FIFO queue (taken from its front,
 * freed blocks join its back in table order), each block counts its
 * references, a sequence gets a new block only when a token starts an
 * unmapped logical block, a token landing in a shared block first gets the
 * writer its own copy (copy-on-write), and a preempted sequence's blocks
 * move to a CPU pool and back (section 4.3; vLLM paper summary, section 5).
 * Every call either succeeds or changes nothing.  A manager is not
 * thread-safe.  Block ids are int32; num_gpu_blocks * block_size must fit
 * int32 (slots do).
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager with empty sequences; gpu_free_order (num_gpu_blocks distinct
 * ids, or NULL for 0, 1, ...) is the initial free queue.  NULL on invalid
 * sizes or allocation failure. */
pa_block_manager* pa_bm_create(int32_t num_gpu_blocks, int32_t num_cpu_blocks,
                               int32_t block_size, const int32_t* gpu_free_order);
void pa_bm_destroy(pa_block_manager* m);

/* A new sequence holding num_tokens tokens: ceil(num_tokens / block_size)
 * blocks.  PA_ERR_SEQUENCE if seq_id exists, PA_ERR_NO_BLOCKS if short. */
int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, int64_t num_tokens);

/* child shares every block of parent (parallel sampling, beam search). */
int pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child);

/* Slot of the sequence's next token (its length grows by one).  copy_pair
 * [2] receives (src, dst) when the token lands in a shared block and the
 * caller must copy src to dst (pa_copy_blocks) before writing, else -1. */
int pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int32_t* slot, int32_t* copy_pair);

/* pa_bm_append_slot for n distinct sequences at once: slots [n] (a decode
 * step's slot_mapping), copy_pairs [n][2] of which *num_copies are used. */
int pa_bm_append_slots(pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t* slots,
                       int32_t* copy_pairs, int32_t* num_copies);

/* Drop a sequence; blocks whose count reaches zero return to the queue. */
int pa_bm_free(pa_block_manager* m, int64_t seq_id);

/* Move a sequence's blocks to the CPU pool (swap_out) or back (swap_in):
 * pairs [k][2] = (from, to) in table order, the copies to perform with
 * pa_copy_blocks before the freed blocks are reused.  A shared GPU block
 * stays for its other users.  max_pairs bounds k (PA_ERR_SHAPE if short). */
int pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int32_t* pairs, int32_t max_pairs,
                   int32_t* num_pairs);
int pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int32_t* pairs, int32_t max_pairs,
                  int32_t* num_pairs);

/* Block tables [n][max_blocks] (padded with -1) and lengths [n] (may be
 * NULL) of n sequences: a batch's block_table and context_lens. */
int pa_bm_block_tables(const pa_block_manager* m, const int64_t* seq_ids, int32_t n,
                       int32_t* tables, int32_t max_blocks, int64_t* lens);

int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id);            /* -1: unknown */
int32_t pa_bm_num_free(const pa_block_manager* m, int32_t on_gpu);
int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block, int32_t on_gpu);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
