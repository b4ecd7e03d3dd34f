// KV cache write: store each new token's K and V into its slot.
//
// The slot of a token is physical_block * block_size + offset: the block
// manager maps the token's logical block (position // block_size) to a
// physical block and the token goes to its position inside it ("How does
// paged attention work (in detail)", section 4.1; vLLM paper summary,
// section 3 "Decoding").  K rows are contiguous in a K tile ([BS][D]); in a
// V tile ([BS/4][D][4]) token t's dim d sits at (t/4*D + d)*4 + t%4.
//
// One wavefront per (group of NQ quads of consecutive tokens, kv head); NQ
// is 1 for a decode step's few tokens and 2 where the grid stays wide.  The
// group's slots are read with one load (a lane per token) and kept in scalar
// registers.  A token quad whose slots are the four slots 4q .. 4q+3 of one
// block, taken by four consecutive tokens (as a prefill chunk's are), is
// written by the wavefront of the group holding its first token; when every
// quad of a group is such a quad, aligned to the group, the wavefront issues
// all of their loads before its first store.  A whole quad takes one store
// instruction per cache tile: the four K rows are 4 D contiguous elements of the K tile and the
// quad's V is 4 D contiguous elements of the V tile, so each lane stores 16
// bytes (8 for fp8) of one contiguous KiB (half a KiB at head size 64 or for
// fp8).  For V, lane l gathers dims 2l, 2l+1 of the four tokens (one 4-byte
// load per token) and interleaves them in registers.  A token whose quad is
// not whole in this call (a decode step's) is written alone: its K row, and
// its V elements one per dim.
//
// fp8 caches store e4m3fn_encode(x * inv_scale) (pa_device.h).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kCwWaves = 4;

template <typename IT>
__device__ __forceinline__ float in_lo16(uint32_t w) {
  if constexpr (__is_same(IT, F16)) return f16_lo(w);
  else return bf16_lo(w);
}
template <typename IT>
__device__ __forceinline__ float in_hi16(uint32_t w) {
  if constexpr (__is_same(IT, F16)) return f16_hi(w);
  else return bf16_hi(w);
}
// fp8 codes of the two 16-bit inputs of w, in bytes 0 and 1
template <typename IT>
__device__ __forceinline__ uint32_t enc2(uint32_t w, float inv) {
  return e4m3fn_encode(in_lo16<IT>(w) * inv) | (e4m3fn_encode(in_hi16<IT>(w) * inv) << 8);
}

template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ const uint16_t* in_row(const CacheWriteParams& p, const void* base,
                                                  int t, int h) {
  return reinterpret_cast<const uint16_t*>(base) + (int64_t)t * p.kv_token_stride + (int64_t)h * D;
}

// The whole quad of tokens t .. t+3 into slots slot .. slot+3 (slot % 4 == 0),
// split into its loads and its stores so that a wavefront can have the loads
// of several quads in flight before it stores the first.
struct QuadRegs {
  u32x4_t k;        // K: lane l holds token l / (D/8), elements 8 (l % (D/8)) .. +7
  uint32_t v[4];    // V: lane l holds dims 2l, 2l+1 of each of the four tokens
};

template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ QuadRegs load_quad(const CacheWriteParams& p, int t, int h, int lane) {
  constexpr int KL = D / 8;                             // lanes per K row (8 elements each)
  QuadRegs r;
  const int tk = lane / KL, ck = lane % KL;
  r.k = *reinterpret_cast<const u32x4_t*>(in_row<IT, CT, D, BS>(p, p.k, t + tk, h) + 8 * ck);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = *reinterpret_cast<const uint32_t*>(in_row<IT, CT, D, BS>(p, p.v, t + i, h) + 2 * lane);
  return r;
}

template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ void store_quad(const CacheWriteParams& p, const QuadRegs& r,
                                           int32_t slot, int h, int lane) {
  const int64_t blk = slot / BS;
  const int off = slot % BS;
  const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)(BS * D);   // elements
  const int64_t kdst = tile + (int64_t)off * D + 8 * lane;          // = row tk, elements 8 ck
  const int64_t vdst = tile + (int64_t)(off >> 2) * 4 * D + 8 * lane;   // dims 2l, 2l+1 x 4 tokens
  const uint32_t* vv = r.v;
  if constexpr (CT::kBytes == 2) {
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p.k_cache) + kdst) = r.k;
    const u32x4_t w = {(vv[0] & 0xFFFFu) | (vv[1] << 16), (vv[2] & 0xFFFFu) | (vv[3] << 16),
                       (vv[0] >> 16) | (vv[1] & 0xFFFF0000u), (vv[2] >> 16) | (vv[3] & 0xFFFF0000u)};
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p.v_cache) + vdst) = w;
  } else {
    const u32x4_t kw = r.k;
    const uint32_t k01 = enc2<IT>(kw[0], p.k_inv_scale), k23 = enc2<IT>(kw[1], p.k_inv_scale);
    const uint32_t k45 = enc2<IT>(kw[2], p.k_inv_scale), k67 = enc2<IT>(kw[3], p.k_inv_scale);
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint8_t*>(p.k_cache) + kdst) =
        u32x2_t{k01 | (k23 << 16), k45 | (k67 << 16)};
    uint32_t c[4];                                      // token i: byte 0 dim 2l, byte 1 dim 2l+1
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = enc2<IT>(vv[i], p.v_inv_scale);
    const uint32_t d0 = (c[0] & 0xFFu) | ((c[1] & 0xFFu) << 8) | ((c[2] & 0xFFu) << 16) |
                        ((c[3] & 0xFFu) << 24);
    const uint32_t d1 = ((c[0] >> 8) & 0xFFu) | (c[1] & 0xFF00u) | ((c[2] & 0xFF00u) << 8) |
                        ((c[3] & 0xFF00u) << 16);
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint8_t*>(p.v_cache) + vdst) = u32x2_t{d0, d1};
  }
}

template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ void write_quad(const CacheWriteParams& p, int t, int32_t slot, int h,
                                           int lane) {
  if (lane >= D / 2) return;                            // 4 D elements, 8 per lane
  store_quad<IT, CT, D, BS>(p, load_quad<IT, CT, D, BS>(p, t, h, lane), slot, h, lane);
}

// Token t alone into slot `slot`: its K row and its V elements one per dim.
template <typename IT, typename CT, int D, int BS>
__device__ __forceinline__ void write_one(const CacheWriteParams& p, int t, int32_t slot, int h,
                                          int lane) {
  if (lane >= D / 2) return;                            // lane l: dims 2l, 2l+1
  const int64_t blk = slot / BS;
  const int off = slot % BS;
  const int64_t tile = (blk * p.num_kv_heads + h) * (int64_t)(BS * D);
  const uint32_t kw = *reinterpret_cast<const uint32_t*>(in_row<IT, CT, D, BS>(p, p.k, t, h) + 2 * lane);
  const uint32_t vw = *reinterpret_cast<const uint32_t*>(in_row<IT, CT, D, BS>(p, p.v, t, h) + 2 * lane);
  const int64_t kdst = tile + (int64_t)off * D + 2 * lane;
  const int64_t vdst = tile + ((int64_t)(off >> 2) * D + 2 * lane) * 4 + (off & 3);
  if constexpr (CT::kBytes == 2) {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.k_cache) + kdst) = kw;
    uint16_t* vc = reinterpret_cast<uint16_t*>(p.v_cache) + vdst;
    vc[0] = (uint16_t)(vw & 0xFFFFu);
    vc[4] = (uint16_t)(vw >> 16);
  } else {
    const uint32_t kc = enc2<IT>(kw, p.k_inv_scale);
    *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(p.k_cache) + kdst) = (uint16_t)kc;
    const uint32_t vc2 = enc2<IT>(vw, p.v_inv_scale);
    uint8_t* vc = reinterpret_cast<uint8_t*>(p.v_cache) + vdst;
    vc[0] = (uint8_t)vc2;
    vc[4] = (uint8_t)(vc2 >> 8);
  }
}

// Wavefront gw takes kv head gw % KVH and the NQ token quads of group
// gw / KVH (tokens 4 NQ g .. 4 NQ g + 4 NQ - 1).
template <typename IT, typename CT, int D, int BS, int NQ>
__global__ __launch_bounds__(64 * kCwWaves) void cache_write_kernel(const CacheWriteParams p) {
  constexpr int NT = 4 * NQ;                            // tokens per wavefront
  const int lane = threadIdx.x & 63;
  // the wavefront's index, uniform: everything below up to the lane offsets
  // stays in scalar registers and the slot reads are independent scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kCwWaves + wave;
  const int T = p.num_tokens;
  const int h = (int)(gw % p.num_kv_heads);
  const int64_t grp = gw / p.num_kv_heads;
  if (grp * NT >= T) return;
  const int t0 = (int)(grp * NT);
  const int64_t pool = p.num_blocks * BS;
  // slots of tokens t0-3 .. t0+NT+2 (-1 outside the call): enough to tell, for
  // each token of the group, whether its quad comes whole.  Lane i reads the
  // slot of token t0-3+i, one load for the wavefront, and each is then moved
  // to a scalar register.
  static_assert(NT + 6 <= 64, "slot window wider than a wavefront");
  int32_t mine = -1;
  {
    const int t = t0 - 3 + lane;
    if (lane < NT + 6 && t >= 0 && t < T) mine = p.slot_mapping[t];
  }
  int32_t sl[NT + 6];
#pragma unroll
  for (int i = 0; i < NT + 6; ++i) sl[i] = __builtin_amdgcn_readlane(mine, i);
  if constexpr (NQ > 1) {
    // every quad of the group whole and aligned to the group (a prefill
    // chunk's): all loads first, then all stores
    bool aligned = true;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int32_t s0 = sl[3 + 4 * q];
      aligned = aligned && s0 >= 0 && s0 + 3 < pool && (s0 & 3) == 0;
#pragma unroll
      for (int i = 1; i < 4; ++i) aligned = aligned && sl[3 + 4 * q + i] == s0 + i;
    }
    if (aligned) {
      if (lane >= D / 2) return;                        // 4 D elements, 8 per lane
      QuadRegs r[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) r[q] = load_quad<IT, CT, D, BS>(p, t0 + 4 * q, h, lane);
#pragma unroll
      for (int q = 0; q < NQ; ++q) store_quad<IT, CT, D, BS>(p, r[q], sl[3 + 4 * q], h, lane);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int32_t slot = sl[3 + j];
    if (slot < 0 || slot >= pool) continue;            // skipped, or outside the pool
    const int k = slot & 3;
    bool whole = true;                                 // quad slots from tokens t-k .. t-k+3
#pragma unroll
    for (int i = 0; i < 4; ++i) whole = whole && sl[3 + j - k + i] == slot - k + i;
    if (whole && k != 0) continue;                     // written with the quad's first token
    if (whole) write_quad<IT, CT, D, BS>(p, t0 + j, slot, h, lane);
    else write_one<IT, CT, D, BS>(p, t0 + j, slot, h, lane);
  }
}

#ifndef PA_CW_QUADS
#define PA_CW_QUADS 2
#endif

template <typename IT, typename CT, int D, int BS, int NQ>
hipError_t launch_nq(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t waves = (int64_t)((p.num_tokens + 4 * NQ - 1) / (4 * NQ)) * p.num_kv_heads;
  const int64_t blocks = (waves + kCwWaves - 1) / kCwWaves;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((cache_write_kernel<IT, CT, D, BS, NQ>), dim3((unsigned)blocks),
                     dim3(64 * kCwWaves), 0, stream, p);
  return hipGetLastError();
}

// Several quads per wavefront only where the grid still holds 16 wavefronts
// per CU (4096): a decode step's few tokens keep one quad per wavefront.
template <typename IT, typename CT, int D, int BS>
hipError_t launch(const CacheWriteParams& p, hipStream_t stream) {
  constexpr int NQ = PA_CW_QUADS;
  const int64_t wide = (int64_t)((p.num_tokens + 4 * NQ - 1) / (4 * NQ)) * p.num_kv_heads;
  if (NQ > 1 && wide >= 4096) return launch_nq<IT, CT, D, BS, NQ>(p, stream);
  return launch_nq<IT, CT, D, BS, 1>(p, stream);
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
