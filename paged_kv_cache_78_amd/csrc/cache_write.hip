// KV cache write: store each new token's K and V into its slot.
//
// The slot of a token is physical_block * block_size + offset: the block
// manager maps the token's logical block (position // block_size) to a
// physical block and the token goes to its position inside it ("How does
// paged attention work (in detail)", section 4.1; vLLM paper summary,
// section 3 "Decoding").  K rows are contiguous in a K tile ([BS][D]); in a
// V tile ([BS/4][D][4]) token t's dim d sits at (t/4*D + d)*4 + t%4.
//
// One thread per (token, kv head, 8 consecutive head dims): a 16-byte load
// of k and of v, one 16-byte (8-byte for fp8) K store and 8 V element stores.
//
// fp8 caches store e4m3fn_encode(x * inv_scale) (pa_device.h).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

template <typename IT>
__device__ __forceinline__ float in_elem(const u32x4_t& w, int j) {
  if constexpr (__is_same(IT, F16)) return (j & 1) ? f16_hi(w[j >> 1]) : f16_lo(w[j >> 1]);
  else return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

template <typename IT, typename CT, int D, int BS>
__global__ __launch_bounds__(256) void cache_write_kernel(const CacheWriteParams p) {
  constexpr int CHUNKS = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * CHUNKS;
  if (gid >= total) return;
  const int c = (int)(gid % CHUNKS);
  const int64_t th = gid / CHUNKS;
  const int h = (int)(th % p.num_kv_heads);
  const int t = (int)(th / p.num_kv_heads);
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / BS;
  const int off = slot % BS;
  if (blk >= p.num_blocks) return;

  const int64_t src = (int64_t)t * p.kv_token_stride + (int64_t)h * D + c * 8;
  const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p.k) + src);
  const u32x4_t vw = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p.v) + src);
  const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)(BS * D);   // elements

  if constexpr (CT::kBytes == 2) {
    uint16_t* kc = reinterpret_cast<uint16_t*>(p.k_cache) + tile + (int64_t)off * D + c * 8;
    *reinterpret_cast<u32x4_t*>(kc) = kw;
    uint16_t* vc = reinterpret_cast<uint16_t*>(p.v_cache) + tile +
                   ((int64_t)(off >> 2) * D + c * 8) * 4 + (off & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = vw[j >> 1];
      vc[(int64_t)j * 4] = (uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
  } else {
    uint32_t kq[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t code = e4m3fn_encode(in_elem<IT>(kw, j) * p.k_inv_scale);
      kq[j >> 2] |= code << (8 * (j & 3));
    }
    uint8_t* kc = reinterpret_cast<uint8_t*>(p.k_cache) + tile + (int64_t)off * D + c * 8;
    *reinterpret_cast<u32x2_t*>(kc) = u32x2_t{kq[0], kq[1]};
    uint8_t* vc = reinterpret_cast<uint8_t*>(p.v_cache) + tile +
                  ((int64_t)(off >> 2) * D + c * 8) * 4 + (off & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vc[(int64_t)j * 4] = (uint8_t)e4m3fn_encode(in_elem<IT>(vw, j) * p.v_inv_scale);
    }
  }
}

template <typename IT, typename CT, int D, int BS>
hipError_t launch(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * (D / 8);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL((cache_write_kernel<IT, CT, D, BS>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename IT, typename CT>
hipError_t pick(const CacheWriteParams& p, int d, int bs, hipStream_t st) {
  if (d == 64) return bs == 16 ? launch<IT, CT, 64, 16>(p, st) : launch<IT, CT, 64, 32>(p, st);
  return bs == 16 ? launch<IT, CT, 128, 16>(p, st) : launch<IT, CT, 128, 32>(p, st);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, Dt in_dt, Dt cache_dt, int head_size,
                              int block_size, hipStream_t stream) {
  if (in_dt == Dt::F16) {
    return cache_dt == Dt::FP8 ? pick<F16, FP8>(p, head_size, block_size, stream)
                               : pick<F16, F16>(p, head_size, block_size, stream);
  }
  return cache_dt == Dt::FP8 ? pick<BF16, FP8>(p, head_size, block_size, stream)
                             : pick<BF16, BF16>(p, head_size, block_size, stream);
}

}  // namespace pa
