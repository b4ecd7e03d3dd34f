// pa_decode_partitioned_noalloc: split-context decode and the merge of its
// partitions in one call, with the partial (max, sum, output) triples kept in
// a static device array of the library instead of caller memory.  For callers
// that cannot allocate device memory.  Nothing here allocates: the array is
// part of the library's code object and is created with it on every device
// the library is loaded on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"

// The partial triples of every call on a device: tmp_out, then max_logits,
// then exp_sums, each starting on a 256-byte boundary.  In host code this
// name is not a device address; kernels only ever see scratch_base()'s.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxReducePartitions = 15360;   // pa_reduce's limit

std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device (null: not looked up)

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_base(void** base) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *base = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_partitioned_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* context_lens, float scale, int32_t num_kv_heads,
    int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t head_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int64_t q_seq_stride, pa_dtype q_dtype,
    pa_dtype cache_dtype, float k_scale, float v_scale, int32_t partition_size,
    int32_t max_context_len, void* stream) {
  if (!out) return PA_ERR_NULL;
  if (((uintptr_t)out & 15u) != 0) return PA_ERR_SHAPE;
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0) return PA_ERR_SHAPE;
  if (partition_size <= 0 || max_context_len < 0) return PA_ERR_WORKSPACE;
  // the three arrays pa_decode_partitioned fills, in 64-bit arithmetic
  const size_t np = ((size_t)max_context_len + partition_size - 1) / partition_size;
  // every check pa_reduce makes is made here or by pa_decode_partitioned,
  // so a launched first half is always followed by the merge
  if (np > (size_t)kMaxReducePartitions) return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_seqs * (size_t)num_heads * np;
  const size_t out_bytes = round256(rows * (size_t)head_size * 4);
  const size_t stat_bytes = round256(rows * 4);
  if (out_bytes + 2 * stat_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  void* base = nullptr;
  const int sb = scratch_base(&base);
  if (sb != PA_OK) return sb;
  float* tmp_out = static_cast<float*>(base);
  float* max_logits = reinterpret_cast<float*>(static_cast<char*>(base) + out_bytes);
  float* exp_sums = reinterpret_cast<float*>(static_cast<char*>(base) + out_bytes + stat_bytes);
  // partitions p < ceil(context_lens[s] / partition_size) are written before
  // they are read, so nothing in the array needs clearing between calls
  const int st = pa_decode_partitioned(q, k_cache, v_cache, block_table, context_lens, scale,
                                       num_kv_heads, block_size, num_seqs, num_heads, head_size,
                                       max_blocks_per_seq, num_blocks, q_seq_stride, q_dtype,
                                       cache_dtype, k_scale, v_scale, partition_size,
                                       max_context_len, tmp_out, max_logits, exp_sums, stream);
  if (st != PA_OK) return st;
  return pa_reduce(out, tmp_out, max_logits, exp_sums, context_lens, num_seqs, num_heads,
                   head_size, partition_size, (int32_t)np, q_dtype, stream);
}
