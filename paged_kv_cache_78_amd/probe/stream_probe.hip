// HBM read-rate probe with the decode kernels' tile stream: random tiles of
// 4 KiB (a 16-bit K or V tile at block size 16, head size 128) or 2 KiB (the
// same in fp8), 16-byte lane loads (one contiguous KiB per load instruction),
// a ring of 2-8 tiles in flight per wavefront, optional non-temporal policy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kWaves = 4;

template <int POLICY>
__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
}

template <int POLICY, int kTileBytes, int kRing>
__global__ __launch_bounds__(64 * kWaves) void stream_probe_kernel(
    const char* pool, int64_t num_tiles, const int32_t* tile_ids, int num_waves,
    int tiles_per_wave, uint32_t* sink) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  const int lane = threadIdx.x & 63;
  constexpr int kLoads = kTileBytes / 1024;
  if (wave >= num_waves) return;
  // the wavefront's tile ids, 64 per VGPR (one per lane), read with
  // v_readlane as the decode kernels read their block tables; loads past the
  // list return 0 and are never used
  const __amdgpu_buffer_rsrc_t idr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(tile_ids + (int64_t)wave * tiles_per_wave), (short)0,
      tiles_per_wave * 4, 0x00020000);
  int cbase = 0;
  int cur = __builtin_amdgcn_raw_buffer_load_b32(idr, lane * 4, 0, 0);
  int nxt = __builtin_amdgcn_raw_buffer_load_b32(idr, (64 + lane) * 4, 0, 0);
  auto tile_of = [&](int i) {   // i increases by one per call
    if (i - cbase == 64) {
      cbase += 64;
      cur = nxt;
      nxt = __builtin_amdgcn_raw_buffer_load_b32(idr, (cbase + 64 + lane) * 4, 0, 0);
    }
    return __builtin_amdgcn_readlane(cur, i - cbase);
  };
  u32x4_t buf[kRing][kLoads];
  // a tile id outside the pool, or a position past the wavefront's list,
  // gets a zero-length descriptor: its loads return zeros and touch nothing
  auto issue = [&](u32x4_t (&d)[kLoads], int i) {
    const int t = i < tiles_per_wave ? tile_of(i) : -1;
    const bool ok = t >= 0 && t < num_tiles;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(pool) + (ok ? (int64_t)t * kTileBytes : 0), (short)0,
        ok ? kTileBytes : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) d[j] = load16<POLICY>(r, lane * 16 + j * 1024);
  };
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) issue(buf[u], u);
  for (int n0 = 0; n0 < tiles_per_wave; n0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      issue(buf[(u + kRing - 1) % kRing], n0 + u + kRing - 1);
      if (n0 + u < tiles_per_wave) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
          x ^= buf[u][j][0] ^ buf[u][j][1] ^ buf[u][j][2] ^ buf[u][j][3];
      }
    }
  }
  sink[(int64_t)wave * 64 + lane] = x;
}


template <int POLICY, int TB>
hipError_t launch_ring(int ring, dim3 grid, hipStream_t st, const char* pool, int64_t num_tiles,
                       const int32_t* ids, int num_waves, int tpw, uint32_t* sink) {
  switch (ring) {
#define PA_PROBE_RING(R)                                                                       \
  case R:                                                                                      \
    hipLaunchKernelGGL((stream_probe_kernel<POLICY, TB, R>), grid, dim3(64 * kWaves), 0, st,   \
                       pool, num_tiles, ids, num_waves, tpw, sink);                            \
    break;
    PA_PROBE_RING(2)
    PA_PROBE_RING(3)
    PA_PROBE_RING(4)
    PA_PROBE_RING(6)
    PA_PROBE_RING(8)
#undef PA_PROBE_RING
  }
  return hipGetLastError();
}

}  // namespace

extern "C" int pa_probe_stream(const void* pool, int64_t num_tiles, const int32_t* tile_ids,
                               int32_t num_waves, int32_t tiles_per_wave, int32_t tile_bytes,
                               int32_t in_flight, int32_t nontemporal, uint32_t* sink,
                               void* stream) {
  if (!pool || !tile_ids || !sink || num_tiles <= 0 || num_waves <= 0 || tiles_per_wave <= 0 ||
      tiles_per_wave > (1 << 24))
    return -2;
  if ((tile_bytes != 2048 && tile_bytes != 4096) ||
      (in_flight != 2 && in_flight != 3 && in_flight != 4 && in_flight != 6 && in_flight != 8))
    return -2;
  const dim3 grid((num_waves + kWaves - 1) / kWaves);
  const char* pl = static_cast<const char*>(pool);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (nontemporal)
    e = tile_bytes == 2048
            ? launch_ring<2, 2048>(in_flight, grid, st, pl, num_tiles, tile_ids, num_waves,
                                   tiles_per_wave, sink)
            : launch_ring<2, 4096>(in_flight, grid, st, pl, num_tiles, tile_ids, num_waves,
                                   tiles_per_wave, sink);
  else
    e = tile_bytes == 2048
            ? launch_ring<0, 2048>(in_flight, grid, st, pl, num_tiles, tile_ids, num_waves,
                                   tiles_per_wave, sink)
            : launch_ring<0, 4096>(in_flight, grid, st, pl, num_tiles, tile_ids, num_waves,
                                   tiles_per_wave, sink);
  return e == hipSuccess ? 0 : -6;
}
