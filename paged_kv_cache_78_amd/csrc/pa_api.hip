// C ABI of libpa: argument validation and kernel selection.  No device code
// lives here; every check happens before anything is launched.
#include <atomic>
#include <math.h>

#include "../../include/pa.h"
#include "pa_kernels.h"

namespace {

using pa::Dt;

constexpr float kLog2eHost = 1.4426950408889634f;
constexpr int kMaxOrderedSeqs = 1024;
// pa_reduce keeps one fp32 weight per partition in LDS (60 KiB at most)
constexpr int kMaxPartitions = 15360;

// Compute units of the current device, asked once per device (256 if the
// runtime cannot say).  Callers on several host threads may ask at once: the
// cache is atomic (they may each ask the runtime; all store the same value).
int compute_units() {
  static std::atomic<int> cache[64];   // 0 = not asked yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The kernels move rows with 16-byte loads and stores.
bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool head_size_ok(int d) { return d == 64 || d == 128; }
bool block_size_ok(int b) { return b == 16 || b == 32; }
bool is16(pa_dtype t) { return t == PA_F16 || t == PA_BF16; }
Dt to_dt(pa_dtype t) { return t == PA_F16 ? Dt::F16 : (t == PA_BF16 ? Dt::BF16 : Dt::FP8); }
bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

int check_cache_types(pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale, float v_scale) {
  if (!is16(q_dtype)) return PA_ERR_DTYPE;
  if (cache_dtype == PA_FP8_E4M3FN) {
    if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_DTYPE;
    return PA_OK;
  }
  return cache_dtype == q_dtype ? PA_OK : PA_ERR_DTYPE;
}

// Shared checks of pa_decode, pa_decode_append and pa_decode_partitioned.
int check_decode(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, const int32_t* context_lens, float scale,
                 int32_t num_kv_heads, int32_t block_size, int32_t num_seqs, int32_t num_heads,
                 int32_t head_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                 int64_t q_seq_stride, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,
                 float v_scale) {
  if (!q || !k_cache || !v_cache || !block_table || !context_lens) return PA_ERR_NULL;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (q_seq_stride < (int64_t)num_heads * head_size || q_seq_stride % 8 != 0) return PA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_SHAPE;   // grid dimension y (partitioned)
  if ((int64_t)num_seqs * num_heads > INT32_MAX) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (!head_size_ok(head_size) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  const int ct = check_cache_types(q_dtype, cache_dtype, k_scale, v_scale);
  if (ct != PA_OK) return ct;
  return PA_OK;
}

pa::DecodeParams make_params(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* context_lens,
                             float scale, int32_t num_kv_heads, int32_t num_seqs,
                             int32_t num_heads, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int64_t q_seq_stride, pa_dtype cache_dtype, float k_scale,
                             float v_scale) {
  pa::DecodeParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.context_lens = context_lens;
  const bool fp8 = cache_dtype == PA_FP8_E4M3FN;
  p.qk_scale_log2 = scale * (fp8 ? k_scale : 1.0f) * kLog2eHost;
  p.v_scale = fp8 ? v_scale : 1.0f;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.q_seq_stride = q_seq_stride;
  p.partition_size = 0;
  p.num_partitions = 1;
  // every workgroup re-derives the order from context_lens: worth it while
  // that scan is short
  p.order_by_length = num_seqs <= kMaxOrderedSeqs ? 1 : 0;
  p.die_order = 0;
  p.num_cus = compute_units();
  return p;
}

// One query head per kv head: vector-ALU kernel.  Grouped heads (G >= 2):
// matrix-core kernel, one wavefront per group.
hipError_t launch_decode(const pa::DecodeParams& p, pa_dtype q_dtype, pa_dtype cache_dtype,
                         int head_size, int block_size, bool partitioned, hipStream_t stream) {
  if (p.num_heads == p.num_kv_heads) {
    return pa::launch_decode_valu(p, to_dt(q_dtype), to_dt(cache_dtype), head_size, block_size,
                                  partitioned, stream);
  }
  return pa::launch_decode_mfma(p, to_dt(q_dtype), to_dt(cache_dtype), head_size, block_size,
                                partitioned, stream);
}

// Device-side address of a pool: device and managed memory as they are,
// pinned host memory through its device mapping.  Pageable host memory (or
// an address the runtime does not know) gives nullptr.  A failed query's
// error is cleared so that it cannot surface at the next launch check.
void* device_address(const void* ptr) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
      return const_cast<void*>(ptr);
    case hipMemoryTypeHost:
      if (!a.devicePointer || !a.hostPointer) return nullptr;
      return reinterpret_cast<char*>(a.devicePointer) +
             (reinterpret_cast<const char*>(ptr) - reinterpret_cast<char*>(a.hostPointer));
    default:
      return nullptr;
  }
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "head size, block size or head grouping not supported";
    case PA_ERR_DTYPE: return "element type combination or fp8 scale not supported";
    case PA_ERR_WORKSPACE: return "invalid partition size or workspace";
    case PA_ERR_HIP: return "the HIP runtime refused the launch";
    case PA_ERR_MEMORY: return "a pointer is not device-accessible memory (device, managed or pinned host)";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_SEQUENCE: return "unknown, duplicate or swapped-out sequence for this call";
    case PA_ERR_SCRATCH: return "the partial results exceed the library's static scratch array";
    default: return "unknown status";
  }
}

int pa_abi_version(void) { return 3; }

int pa_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                   const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                   int32_t head_size, int32_t block_size, int64_t num_blocks,
                   int64_t kv_token_stride, pa_dtype in_dtype, pa_dtype cache_dtype,
                   float k_scale, float v_scale, void* stream) {
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (kv_token_stride < (int64_t)num_kv_heads * head_size || kv_token_stride % 8 != 0)
    return PA_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_SHAPE;
  if (!head_size_ok(head_size) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const int ct = check_cache_types(in_dtype, cache_dtype, k_scale, v_scale);
  if (ct != PA_OK) return ct;
  if (num_tokens == 0) return PA_OK;
  pa::CacheWriteParams p{};
  p.k = k;
  p.v = v;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.num_blocks = num_blocks;
  p.kv_token_stride = kv_token_stride;
  const bool fp8 = cache_dtype == PA_FP8_E4M3FN;
  p.k_inv_scale = fp8 ? 1.0f / k_scale : 1.0f;
  p.v_inv_scale = fp8 ? 1.0f / v_scale : 1.0f;
  const hipError_t e = pa::launch_cache_write(p, to_dt(in_dtype), to_dt(cache_dtype), head_size,
                                              block_size, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens, float scale,
              int32_t num_kv_heads, int32_t block_size, int32_t num_seqs, int32_t num_heads,
              int32_t head_size, int32_t max_blocks_per_seq, int64_t num_blocks,
              int64_t q_seq_stride, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,
              float v_scale, void* stream) {
  if (!out) return PA_ERR_NULL;
  const int st = check_decode(q, k_cache, v_cache, block_table, context_lens, scale,
                              num_kv_heads, block_size, num_seqs, num_heads, head_size,
                              max_blocks_per_seq, num_blocks, q_seq_stride, q_dtype, cache_dtype,
                              k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!aligned16(out)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  pa::DecodeParams p = make_params(q, k_cache, v_cache, block_table, context_lens, scale,
                                   num_kv_heads, num_seqs, num_heads, max_blocks_per_seq,
                                   num_blocks, q_seq_stride, cache_dtype, k_scale, v_scale);
  p.out = out;
  const hipError_t e =
      launch_decode(p, q_dtype, cache_dtype, head_size, block_size, false, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_decode_append(void* out, const void* q, const void* k, const void* v, void* k_cache,
                     void* v_cache, const int32_t* slot_mapping, const int32_t* block_table,
                     const int32_t* context_lens, float scale, int32_t num_kv_heads,
                     int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t head_size,
                     int32_t max_blocks_per_seq, int64_t num_blocks, int64_t q_seq_stride,
                     int64_t kv_token_stride, pa_dtype q_dtype, pa_dtype cache_dtype,
                     float k_scale, float v_scale, void* stream) {
  if (!out || !k || !v || !slot_mapping) return PA_ERR_NULL;
  const int st = check_decode(q, k_cache, v_cache, block_table, context_lens, scale,
                              num_kv_heads, block_size, num_seqs, num_heads, head_size,
                              max_blocks_per_seq, num_blocks, q_seq_stride, q_dtype, cache_dtype,
                              k_scale, v_scale);
  if (st != PA_OK) return st;
  if (kv_token_stride < (int64_t)num_kv_heads * head_size || kv_token_stride % 8 != 0)
    return PA_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(k) || !aligned16(v)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  pa::DecodeParams p = make_params(q, k_cache, v_cache, block_table, context_lens, scale,
                                   num_kv_heads, num_seqs, num_heads, max_blocks_per_seq,
                                   num_blocks, q_seq_stride, cache_dtype, k_scale, v_scale);
  p.out = out;
  p.append = 1;
  p.k_new = k;
  p.v_new = v;
  p.slot_mapping = slot_mapping;
  p.kv_token_stride = kv_token_stride;
  const bool fp8 = cache_dtype == PA_FP8_E4M3FN;
  p.k_inv_scale = fp8 ? 1.0f / k_scale : 1.0f;
  p.v_inv_scale = fp8 ? 1.0f / v_scale : 1.0f;
  const hipError_t e =
      launch_decode(p, q_dtype, cache_dtype, head_size, block_size, false, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* block_mapping, int32_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int32_t num_kv_heads, int32_t head_size,
                   int32_t block_size, pa_dtype cache_dtype, void* stream) {
  if (!src_k || !src_v || !dst_k || !dst_v || (num_pairs > 0 && !block_mapping))
    return PA_ERR_NULL;
  if (num_pairs < 0 || num_pairs > 65535 || src_num_blocks <= 0 || dst_num_blocks <= 0 ||
      num_kv_heads <= 0 || head_size <= 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (!head_size_ok(head_size) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (cache_dtype != PA_F16 && cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3FN)
    return PA_ERR_DTYPE;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  pa::BlockCopyParams p{};
  p.src_k = device_address(src_k);
  p.src_v = device_address(src_v);
  p.dst_k = device_address(dst_k);
  p.dst_v = device_address(dst_v);
  p.mapping = static_cast<const int32_t*>(device_address(block_mapping));
  if (!p.src_k || !p.src_v || !p.dst_k || !p.dst_v || !p.mapping) return PA_ERR_MEMORY;
  p.num_pairs = num_pairs;
  p.src_num_blocks = src_num_blocks;
  p.dst_num_blocks = dst_num_blocks;
  p.block_bytes = (int64_t)num_kv_heads * block_size * head_size *
                  (cache_dtype == PA_FP8_E4M3FN ? 1 : 2);
  const hipError_t e = pa::launch_copy_blocks(p, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* cu_seqlens_q,
               const int32_t* context_lens, float scale, int32_t num_kv_heads,
               int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t head_size,
               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t total_q,
               int32_t max_seqlen_q, int64_t q_token_stride, int32_t causal, pa_dtype q_dtype,
               pa_dtype cache_dtype, float k_scale, float v_scale, void* stream) {
  if (!out || !cu_seqlens_q) return PA_ERR_NULL;
  const int st = check_decode(q, k_cache, v_cache, block_table, context_lens, scale,
                              num_kv_heads, block_size, num_seqs, num_heads, head_size,
                              max_blocks_per_seq, num_blocks, q_token_stride, q_dtype, cache_dtype,
                              k_scale, v_scale);
  if (st != PA_OK) return st;
  if (total_q < 0 || max_seqlen_q < 0 || num_kv_heads > 65535) return PA_ERR_SHAPE;
  if (!aligned16(out)) return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  pa::PrefillParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.cu_seqlens_q = cu_seqlens_q;
  p.context_lens = context_lens;
  const bool fp8 = cache_dtype == PA_FP8_E4M3FN;
  p.qk_scale_log2 = scale * (fp8 ? k_scale : 1.0f) * kLog2eHost;
  p.v_scale = fp8 ? v_scale : 1.0f;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.q_token_stride = q_token_stride;
  p.total_q = total_q;
  p.max_seqlen_q = max_seqlen_q;
  p.causal = causal ? 1 : 0;
  const hipError_t e = pa::launch_prefill(p, to_dt(q_dtype), to_dt(cache_dtype), head_size,
                                          block_size, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_partition_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                    int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0 || max_context_len < 0 ||
      partition_size <= 0)
    return 0;
  const int64_t np = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  const int64_t rows = (int64_t)num_seqs * num_heads * np;
  return (size_t)(rows * head_size * 4 + 2 * rows * 4);
}

int pa_decode_partitioned(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* context_lens, float scale,
                          int32_t num_kv_heads, int32_t block_size, int32_t num_seqs,
                          int32_t num_heads, int32_t head_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, int64_t q_seq_stride, pa_dtype q_dtype,
                          pa_dtype cache_dtype, float k_scale, float v_scale,
                          int32_t partition_size, int32_t max_context_len, float* tmp_out,
                          float* max_logits, float* exp_sums, void* stream) {
  const int st = check_decode(q, k_cache, v_cache, block_table, context_lens, scale,
                              num_kv_heads, block_size, num_seqs, num_heads, head_size,
                              max_blocks_per_seq, num_blocks, q_seq_stride, q_dtype, cache_dtype,
                              k_scale, v_scale);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % block_size != 0 || max_context_len < 0)
    return PA_ERR_WORKSPACE;
  if (!tmp_out || !max_logits || !exp_sums) return PA_ERR_NULL;
  if (!aligned16(tmp_out)) return PA_ERR_SHAPE;
  const int64_t np = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  if (np > 65535) return PA_ERR_WORKSPACE;   // grid dimension z
  if (num_seqs == 0 || np == 0) return PA_OK;
  pa::DecodeParams p = make_params(q, k_cache, v_cache, block_table, context_lens, scale,
                                   num_kv_heads, num_seqs, num_heads, max_blocks_per_seq,
                                   num_blocks, q_seq_stride, cache_dtype, k_scale, v_scale);
  p.tmp_out = tmp_out;
  p.max_logits = max_logits;
  p.exp_sums = exp_sums;
  p.partition_size = partition_size;
  p.num_partitions = (int32_t)np;
  const hipError_t e =
      launch_decode(p, q_dtype, cache_dtype, head_size, block_size, true, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_reduce(void* out, const float* tmp_out, const float* max_logits, const float* exp_sums,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
              int32_t head_size, int32_t partition_size, int32_t max_num_partitions,
              pa_dtype out_dtype, void* stream) {
  if (!out || !context_lens) return PA_ERR_NULL;
  if (max_num_partitions > 0 && (!tmp_out || !max_logits || !exp_sums)) return PA_ERR_NULL;
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_SHAPE;
  if (!aligned16(out) || (max_num_partitions > 0 && !aligned16(tmp_out))) return PA_ERR_SHAPE;
  if (partition_size <= 0 || max_num_partitions < 0 || max_num_partitions > kMaxPartitions)
    return PA_ERR_WORKSPACE;
  if (!head_size_ok(head_size)) return PA_ERR_UNSUPPORTED;
  if (!is16(out_dtype)) return PA_ERR_DTYPE;
  if (num_seqs == 0) return PA_OK;
  pa::ReduceParams p{};
  p.out = out;
  p.tmp_out = tmp_out;
  p.max_logits = max_logits;
  p.exp_sums = exp_sums;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.partition_size = partition_size;
  p.max_num_partitions = max_num_partitions;
  const hipError_t e = pa::launch_reduce(p, to_dt(out_dtype), head_size, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
