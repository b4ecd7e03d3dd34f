// KV cache write: store each new token's K and V into its slot.
//
// The slot of a token is physical_block * block_size + offset: the block
// manager maps the token's logical block (position // block_size) to a
// physical block and the token goes to its position inside it ("How does
// paged attention work (in detail)", section 4.1; vLLM paper summary,
// section 3 "Decoding").  K rows are contiguous in a K tile ([BS][D]); in a
// V tile ([BS/4][D][4]) token t's dim d sits at (t/4*D + d)*4 + t%4.
//
// One thread per (group of 4 tokens, kv head, 8 consecutive head dims).
// Tokens whose slots fill a whole token quad of a block (slots 4q .. 4q+3
// from consecutive tokens, as a prefill chunk's do) are written by the
// thread of the quad's first token: four K rows, and the quad's V for its 8
// dims as 4 tokens x 8 dims transposed in registers into 64 contiguous bytes
// (32 for fp8), so V is stored in 16-byte pieces.  Any other token (a quad
// only partly in this call, as a decode step's) is written alone: one
// 16-byte (8-byte for fp8) K store and 8 V element stores.
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

// Token t's K/V (n = 4: tokens t .. t+3, a whole quad) into slot `slot`
// (n = 4: the quad's first slot), kv head h, dims 8c .. 8c+7.
template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ void write_tokens(const CacheWriteParams& p, int t, int n, int32_t slot,
                                             int h, int c) {
  const int64_t blk = slot / BS;
  const int off = slot % BS;
  const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)(BS * D);   // elements
  u32x4_t kw[4], vw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < n) {
      const int64_t src = (int64_t)(t + i) * p.kv_token_stride + (int64_t)h * D + c * 8;
      kw[i] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p.k) + src);
      vw[i] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p.v) + src);
    }
  }
  if constexpr (CT::kBytes == 2) {
    uint16_t* kc = reinterpret_cast<uint16_t*>(p.k_cache) + tile + (int64_t)off * D + c * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < n) *reinterpret_cast<u32x4_t*>(kc + (int64_t)i * D) = kw[i];
    uint16_t* vc = reinterpret_cast<uint16_t*>(p.v_cache) + tile +
                   ((int64_t)(off >> 2) * D + c * 8) * 4 + (off & 3);
    if (n == 4) {
      // dims 2 q2, 2 q2 + 1 of the 4 tokens -> 16 bytes at vc + 8 q2 (tokens in order)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t a0 = vw[0][q2], a1 = vw[1][q2], a2 = vw[2][q2], a3 = vw[3][q2];
        const u32x4_t w = {(a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16),
                           (a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u)};
        *reinterpret_cast<u32x4_t*>(vc + 8 * q2) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = vw[0][j >> 1];
        vc[(int64_t)j * 4] = (uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
    }
  } else {
    uint8_t* kc = reinterpret_cast<uint8_t*>(p.k_cache) + tile + (int64_t)off * D + c * 8;
    uint32_t vq[4][2];                                 // token i's 8 V codes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < n) {
        uint32_t kq[2] = {0u, 0u};
        vq[i][0] = vq[i][1] = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kq[j >> 2] |= e4m3fn_encode(in_elem<IT>(kw[i], j) * p.k_inv_scale) << (8 * (j & 3));
          vq[i][j >> 2] |= e4m3fn_encode(in_elem<IT>(vw[i], j) * p.v_inv_scale) << (8 * (j & 3));
        }
        *reinterpret_cast<u32x2_t*>(kc + (int64_t)i * D) = u32x2_t{kq[0], kq[1]};
      }
    }
    uint8_t* vc = reinterpret_cast<uint8_t*>(p.v_cache) + tile +
                  ((int64_t)(off >> 2) * D + c * 8) * 4 + (off & 3);
    if (n == 4) {
      // dim j of the 4 tokens -> 4 bytes at vc + 4 j
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = 8 * (j & 3);
        w[j] = ((vq[0][j >> 2] >> sh) & 0xFFu) | (((vq[1][j >> 2] >> sh) & 0xFFu) << 8) |
               (((vq[2][j >> 2] >> sh) & 0xFFu) << 16) | (((vq[3][j >> 2] >> sh) & 0xFFu) << 24);
      }
      *reinterpret_cast<u32x4_t*>(vc) = u32x4_t{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4_t*>(vc + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) vc[(int64_t)j * 4] = (uint8_t)(vq[0][j >> 2] >> (8 * (j & 3)));
    }
  }
}

template <typename IT, typename CT, int D, int BS>
__global__ __launch_bounds__(256) void cache_write_kernel(const CacheWriteParams p) {
  constexpr int CHUNKS = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int T = p.num_tokens;
  const int64_t total = (int64_t)((T + 3) / 4) * p.num_kv_heads * CHUNKS;
  if (gid >= total) return;
  const int c = (int)(gid % CHUNKS);
  const int64_t th = gid / CHUNKS;
  const int h = (int)(th % p.num_kv_heads);
  const int t0 = 4 * (int)(th / p.num_kv_heads);
  const int64_t pool = p.num_blocks * BS;
  // slots of tokens t0-3 .. t0+6 (one load each, issued together; -1 outside
  // the call): enough to tell, for each of the group's tokens, whether its
  // quad comes whole
  int32_t sl[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int t = t0 - 3 + i;
    sl[i] = (t >= 0 && t < T) ? p.slot_mapping[t] : -1;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t slot = sl[3 + j];
    if (slot < 0 || slot >= pool) continue;            // skipped, or outside the pool
    const int k = slot & 3;
    bool whole = true;                                 // quad slots from tokens t-k .. t-k+3
#pragma unroll
    for (int i = 0; i < 4; ++i) whole = whole && sl[3 + j - k + i] == slot - k + i;
    if (whole && k != 0) continue;                     // written by the quad's first token
    write_tokens<IT, CT, D, BS>(p, t0 + j, whole ? 4 : 1, slot, h, c);
  }
}

template <typename IT, typename CT, int D, int BS>
hipError_t launch(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)((p.num_tokens + 3) / 4) * p.num_kv_heads * (D / 8);
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
