// Varlen / chunked prefill attention over the paged cache, on the gfx950
// matrix cores.
//
// Method ("Paged attention" wiki of a continuous-batching library, Varlen
// path: the query tokens of all sequences are packed and assigned to their
// sequence by cumulative lengths; vLLM "Paged Attention" design page, QK /
// Softmax / LV: scores, a stable softmax and the weighted V sum).  Sequence s
// has n_s query tokens (q rows cu[s] .. cu[s+1]-1) and K_s tokens in the
// cache, the queries being its last n_s positions: query i sits at position
// K_s - n_s + i and, causal, attends keys 0 .. K_s - n_s + i.
//
// Layout of the work: the n_s * G query rows of (sequence, kv head) (G query
// heads per kv head, row r = token r / G, head r % G) are cut into blocks of
// 16 rows.  A wavefront owns one block: the 16 rows are the 16 columns of
//
//   S^T [16 tokens x 16 rows] = K [16 x D] . Q^T [D x 16]      (v_mfma 16x16x32)
//   O^T [D x 16 rows]        += V^T [D x 16] . P^T [16 x 16]   (v_mfma 16x16x16)
//
// exactly as in the decode kernel for a group of heads, with one online
// softmax per column and a per-column causal limit.  The wavefront streams
// the key tiles up to the largest limit of its columns through the block
// table; four wavefronts (64 rows) share a workgroup, so a tile they all read
// comes from the same L2 lines.  Weight precision, fp8 decoding and masking
// follow the decode kernel: P in f16 (f16 and fp8 caches) or split into two
// bf16 parts (bf16 caches); keys past a column's limit get a -inf logit and
// a zero weight, and V rows past the context are zeroed before the product.
#include <type_traits>

#include "mfma_common.h"
#include "pa_decode_common.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kRowsPerWg = 16 * kPrefillWaves;
constexpr int kPrefillNbuf = 3;
constexpr float kNegInfP = kMfmaNegInf;
constexpr float kSlackP = 8.0f;

template <typename QT, typename CT, int D, int BS, bool CAUSAL>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_mfma_kernel(const PrefillParams p) {
  constexpr int ESZ = CT::kBytes;
  constexpr int SUB = BS / 16;
  constexpr int TILE_BYTES = BS * D * ESZ;
  constexpr int NQK = D / 32;
  constexpr int NPV = D / 16;
  constexpr int E = 16 / (4 * ESZ);
  constexpr int NVL = NPV / E;
  constexpr int NKL = ESZ == 2 ? NQK : NQK / 2;
  constexpr int NBUF = kPrefillNbuf;
  using M = Mma<QT>;
  using MV = std::conditional_t<ESZ == 1, Mma<F16>, Mma<QT>>;
  constexpr bool kSplitP = ESZ == 2 && __is_same(QT, BF16);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;          // query row (column of the products)
  const int g = lane >> 4;          // lane group
  const int s = blockIdx.y;
  const int kvh = blockIdx.z;
  const int H = p.num_heads;
  const int KVH = p.num_kv_heads;
  const int G = H / KVH;
  const int MB = p.max_blocks_per_seq;

  const int32_t q0 = p.cu_seqlens_q[s];
  const int32_t q1 = p.cu_seqlens_q[s + 1];
  const int nq = q1 - q0;
  // packed rows outside [0, total_q) are never touched
  if (q0 < 0 || q1 > p.total_q || nq <= 0) return;
  const int rows = nq * G;
  if ((int)blockIdx.x * kRowsPerWg >= rows) return;
  const int row = (int)blockIdx.x * kRowsPerWg + wave * 16 + n;
  const bool row_ok = row < rows;
  const int qi = row_ok ? row / G : 0;             // query token within the chunk
  const int h = kvh * G + (row_ok ? row % G : 0);
  const int K = p.context_lens[s];
  const bool bad_len = K < 0 || K > MB * BS || nq > p.max_seqlen_q;
  // keys this row attends: positions 0 .. lim-1
  int lim = 0;
  if (row_ok && !bad_len) lim = CAUSAL ? min(K, K - nq + qi + 1) : K;
  lim = max(lim, 0);
  int wl = lim;                                     // the wavefront's largest limit
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) wl = max(wl, __shfl_xor(wl, o, 64));
  const int ntiles = __builtin_amdgcn_readfirstlane((wl + BS - 1) / BS);
  const int last_tile = (K + BS - 1) / BS - 1;      // the sequence's last (partial) tile
  const int last_len = K - last_tile * BS;

  auto write_out = [&](const float4_t (&o)[NPV]) {
    if (!row_ok) return;
    uint16_t* dst0 = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)(q0 + qi) * H + h) * D;
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      float run[4 * E];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) run[E * r + e] = o[E * i + e][r];
      uint16_t* dst = dst0 + 16 * E * i + 4 * E * g;
#pragma unroll
      for (int c = 0; c < E / 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (uint32_t)to_bits16<QT>(run[8 * c + 2 * k]) |
                 ((uint32_t)to_bits16<QT>(run[8 * c + 2 * k + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(dst + 8 * c) = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
  };

  if (bad_len) {
    float4_t o[NPV];
    const float nanv = __builtin_nanf("");
#pragma unroll
    for (int j = 0; j < NPV; ++j) o[j] = float4_t{nanv, nanv, nanv, nanv};
    write_out(o);
    return;
  }

  // Q^T operand: row n's query token and head, dims in the QK chunk order
  u32x4_t qb[NQK];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       ((int64_t)(q0 + qi) * p.q_token_stride + (int64_t)h * D) * 2;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      qb[c] = row_ok ? *reinterpret_cast<const u32x4_t*>(qrow + qk_dim<ESZ>(c, g) * 2)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE_BYTES;
  const int64_t block_stride = (int64_t)KVH * TILE_BYTES;
  TableWindow tw;
  tw.init(p.block_table + (int64_t)s * MB, ntiles, p.num_blocks, lane);

  uint32_t koff[SUB][NKL];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int i = 0; i < NKL; ++i)
      koff[u][i] = (uint32_t)((16 * u + n) * D * ESZ +
                              (ESZ == 2 ? qk_dim<2>(i, g) * 2 : 64 * i + 16 * g));
  uint32_t voff[SUB][NVL];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int i = 0; i < NVL; ++i)
      voff[u][i] = (uint32_t)(((4 * u + g) * D + E * (16 * i + n)) * 4 * ESZ);

  u32x4_t kb[NBUF][SUB][NKL];
  u32x4_t vb[NBUF][SUB][NVL];

  auto issue = [&](u32x4_t (&kd)[SUB][NKL], u32x4_t (&vd)[SUB][NVL], int t) {
    int phys = 0;
    uint32_t bytes = 0;
    if (t < ntiles) {
      phys = tw.phys(t, lane);
      bytes = TILE_BYTES;
    }
    const int64_t off = (int64_t)phys * block_stride;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int i = 0; i < NKL; ++i) kd[u][i] = buffer_load16(rk, koff[u][i]);
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int i = 0; i < NVL; ++i) vd[u][i] = buffer_load16(rv, voff[u][i]);
  };

  float m = kNegInfP;
  float l = 0.0f;
  float4_t acc[NPV];
#pragma unroll
  for (int j = 0; j < NPV; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto k_operand = [&](const u32x4_t (&kd)[NKL], int c) -> u32x4_t {
    if constexpr (ESZ == 2) {
      return kd[c];
    } else {
      const u32x4_t w = kd[c >> 1];
      const uint32_t a = (c & 1) ? w[2] : w[0];
      const uint32_t b = (c & 1) ? w[3] : w[1];
      return u32x4_t{M::template fp8x2<false>(a), M::template fp8x2<true>(a),
                     M::template fp8x2<false>(b), M::template fp8x2<true>(b)};
    }
  };
  auto v_operand = [&](const u32x4_t& w, int e) -> u32x2_t {
    if constexpr (ESZ == 2) {
      return u32x2_t{w[2 * e], w[2 * e + 1]};
    } else {
      const uint32_t v = w[e];
      return u32x2_t{MV::template fp8x2<false>(v), MV::template fp8x2<true>(v)};
    }
  };

  // tile t: keys t*BS + 16u + 4g + r for column n
  auto process = [&](const u32x4_t (&kd)[SUB][NKL], const u32x4_t (&vd)[SUB][NVL], int t) {
    const bool vmask = (t == last_tile) && (last_len < BS);   // V rows past the context
    const bool kmask = (t + 1) * BS > lim;                    // some key past this column's limit
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      float4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NQK; ++c) sc = M::qk(k_operand(kd[u], c), qb[c], sc);
      float x[4];
      bool ok[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ok[r] = !kmask || (t * BS + 16 * u + 4 * g + r) < lim;
        x[r] = ok[r] ? sc[r] * p.qk_scale_log2 : kNegInfP;
      }
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (__builtin_amdgcn_ballot_w64(mt > m + kSlackP) != 0) {
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m, mt);
        const float alpha = (m == mn) ? 1.0f : exp2_hw(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int j = 0; j < NPV; ++j) acc[j] *= alpha;
      }
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = ok[r] ? exp2_hw(x[r] - m) : 0.0f;
      const uint32_t p01 = MV::pack(pr[0], pr[1]);
      const uint32_t p23 = MV::pack(pr[2], pr[3]);
      u32x2_t pl = {0u, 0u};
      if constexpr (kSplitP) {
        pl = u32x2_t{MV::pack(pr[0] - MV::lo(p01), pr[1] - MV::hi(p01)),
                     MV::pack(pr[2] - MV::lo(p23), pr[3] - MV::hi(p23))};
        l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      } else {
        l += (MV::lo(p01) + MV::hi(p01)) + (MV::lo(p23) + MV::hi(p23));
      }
      const u32x2_t pb = {p01, p23};
      uint32_t keep0 = 0xFFFFFFFFu, keep1 = 0xFFFFFFFFu;
      if (vmask) {
        const int t0 = 16 * u + 4 * g;
        keep0 = (t0 + 0 < last_len ? 0x0000FFFFu : 0u) | (t0 + 1 < last_len ? 0xFFFF0000u : 0u);
        keep1 = (t0 + 2 < last_len ? 0x0000FFFFu : 0u) | (t0 + 3 < last_len ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        u32x2_t a = v_operand(vd[u][j / E], j % E);
        if (vmask) a = u32x2_t{a[0] & keep0, a[1] & keep1};
        acc[j] = MV::pv(a, pb, acc[j]);
      }
      if constexpr (kSplitP) {
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
          u32x2_t a = v_operand(vd[u][j / E], j % E);
          if (vmask) a = u32x2_t{a[0] & keep0, a[1] & keep1};
          acc[j] = MV::pv(a, pl, acc[j]);
        }
      }
    }
  };

#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(kb[u], vb[u], u);
  for (int t0 = 0; t0 < ntiles; t0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int t = t0 + u;
      issue(kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF], t + NBUF - 1);
      if (t < ntiles) process(kb[u], vb[u], t);
    }
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // a row with no key gives zeros; a bad table entry NaN
  const float inv = tw.bad ? __builtin_nanf("") : (l > 0.0f ? p.v_scale / l : 0.0f);
  float4_t o[NPV];
#pragma unroll
  for (int j = 0; j < NPV; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[j][r] = acc[j][r] * inv;
  write_out(o);
}

template <typename QT, typename CT, int D, int BS>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const int G = p.num_heads / p.num_kv_heads;
  const int64_t rows = (int64_t)p.max_seqlen_q * G;
  const unsigned bx = (unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg);
  const dim3 grid(bx, p.num_seqs, p.num_kv_heads);
  if (p.causal)
    hipLaunchKernelGGL((prefill_mfma_kernel<QT, CT, D, BS, true>), grid, dim3(64 * kPrefillWaves),
                       0, stream, p);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<QT, CT, D, BS, false>), grid,
                       dim3(64 * kPrefillWaves), 0, stream, p);
  return hipGetLastError();
}

template <typename QT, typename CT>
hipError_t pick(const PrefillParams& p, int d, int bs, hipStream_t st) {
  if (d == 64) return bs == 16 ? launch_one<QT, CT, 64, 16>(p, st) : launch_one<QT, CT, 64, 32>(p, st);
  return bs == 16 ? launch_one<QT, CT, 128, 16>(p, st) : launch_one<QT, CT, 128, 32>(p, st);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, Dt q_dt, Dt cache_dt, int head_size,
                          int block_size, hipStream_t stream) {
  if (q_dt == Dt::F16) {
    return cache_dt == Dt::FP8 ? pick<F16, FP8>(p, head_size, block_size, stream)
                               : pick<F16, F16>(p, head_size, block_size, stream);
  }
  return cache_dt == Dt::FP8 ? pick<BF16, FP8>(p, head_size, block_size, stream)
                             : pick<BF16, BF16>(p, head_size, block_size, stream);
}

}  // namespace pa
