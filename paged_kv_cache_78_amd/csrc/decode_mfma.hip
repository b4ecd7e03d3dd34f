// Paged decode attention for grouped query heads (2 <= G <= 16 query heads per
// kv head) on the gfx950 matrix cores.
//
// Method (vLLM "Paged Attention" design page, sections "QK", "Softmax",
// "Value", "LV", "Output"; the group of query heads that share one kv head
// is named there through num_kv_heads / kv_head_idx): per (sequence, kv head
// [, partition]) the G query heads of the group all read the same K/V tiles,
// so the scores and the weighted value sum are dense contractions:
//
//   S^T [16 tokens x 16 heads] = K [16 x D] . Q^T [D x 16]     (v_mfma 16x16x32)
//   O^T [D x 16 heads]        += V^T [D x 16] . P^T [16 x 16]   (v_mfma 16x16x16)
//
// One 64-lane wavefront per (sequence, kv head[, partition]), 16-token
// sub-tiles (a block of 32 tokens is two sub-tiles).  Operand layouts:
//  * A = K: lane l holds token l%16 and 8 consecutive head dims; the dims of
//    the 32-wide k-chunks are chosen so each lane's 16-byte load is one
//    contiguous piece of the token's row.  Q^T (B) uses the same dim order.
//  * S^T lands with lane l holding head l%16 and tokens 4(l/16)..+3: exactly
//    the B-operand layout P^T needs for the second product, and the per-head
//    softmax state (max, rescale factor) lives in the lanes of that head's
//    output column.
//  * A = V^T: lane l holds head dim 16j + l%16 and tokens 4(l/16)..+3, an
//    8-byte piece of the dim-major V tile row (4 bytes for fp8).
//  * P goes into the product as f16 (f16 and fp8 caches; the softmax sum
//    adds the same rounded weights) or, for bf16 caches, split into two bf16
//    parts hi + lo with one product each (16 bits of every weight).
//  * fp8 e4m3fn K/V convert exactly to the q type (QK) and to f16 (PV)
//    before the products; the cache scales multiply the logits (k_scale) and
//    the output (v_scale).
//  * The per-head max over a sub-tile's 16 tokens needs two cross-row
//    exchanges; everything else stays in registers.  Tokens past the context
//    get -inf logits and zeroed V operands (a NaN in an unused slot must not
//    reach the matrix product).
// The block table, prefetch pipeline and error handling follow the
// one-head-per-kv-head kernel.
#include <type_traits>

#include "mfma_common.h"
#include "pa_decode_common.h"
#include "pa_kernels.h"

#ifndef PA_MFMA_NBUF
#define PA_MFMA_NBUF 3
#endif
// fp8 caches: tiles in flight per wavefront and wavefronts per SIMD
#ifndef PA_MFMA_NBUF_FP8
#define PA_MFMA_NBUF_FP8 3
#endif
#ifndef PA_MFMA_FP8_WAVES_PER_EU
#define PA_MFMA_FP8_WAVES_PER_EU 3
#endif
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif

namespace pa {
namespace {

constexpr float kNegInf = kMfmaNegInf;

// fp8 caches: three wavefronts per SIMD fit without spilling (16-bit caches
// need the register budget of two), and the extra wavefronts keep more tiles
// in flight per compute unit.
template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(CT::kBytes == 1 ? PA_MFMA_FP8_WAVES_PER_EU : 1)))
void decode_mfma_kernel(const DecodeParams p) {
  constexpr int ESZ = CT::kBytes;
  constexpr int SUB = BS / 16;              // 16-token sub-tiles per block
  constexpr int TILE_BYTES = BS * D * ESZ;
  constexpr int NQK = D / 32;               // QK products per sub-tile
  constexpr int NPV = D / 16;               // PV products per sub-tile
  constexpr int E = 16 / (4 * ESZ);         // head dims per 16-byte V load (4 tokens each)
  constexpr int NVL = NPV / E;              // 16-byte V loads per sub-tile
  constexpr int NKL = ESZ == 2 ? NQK : NQK / 2;   // 16-byte K loads per sub-tile
  // fp8 tiles in flight: three of 16 tokens, two of 32 (64 tokens, and no
  // spills under the fp8 occupancy's register budget)
  constexpr int NBUF = ESZ == 1 ? (BS == 32 ? 2 : PA_MFMA_NBUF_FP8) : PA_MFMA_NBUF;
  static_assert(BS % 16 == 0 && D % 64 == 0, "shape");
  using M = Mma<QT>;
  // PV operand type: f16 for fp8 caches (decoded e4m3fn is exact in f16,
  // which keeps 11 bits of each weight), else the cache's own type.  With
  // bf16 the weights are split as P = hi + lo, two bf16 values, and PV runs
  // once per part: a single bf16 weight carries 8 bits, too few for the
  // output tolerance on short contexts with widely spread V values.
  using MV = std::conditional_t<ESZ == 1, Mma<F16>, Mma<QT>>;
  constexpr bool kSplitP = ESZ == 2 && __is_same(QT, BF16);

  // WAVES wavefronts share one (sequence, kv head[, partition]): wavefront w
  // takes the w-th contiguous share of its tiles; the states merge in LDS.
  constexpr int NSTATE = NPV * 4 + 4;       // floats of one lane's softmax state
  __shared__ int s_hist[PART ? 1 : WAVES * kSchedKeys];
  __shared__ float s_state[WAVES > 1 ? (WAVES - 1) * kWave * NSTATE : 1];
  __shared__ __attribute__((aligned(16))) float s_new[PART ? 4 : 2 * D];   // fused append
  __shared__ uint16_t s_new_bits[PART ? 2 : 2 * D];
  __shared__ int s_table[table_lds_ints(WAVES)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;          // head column / token row of the products
  const int g = lane >> 4;          // lane group: k-block / row block
  const int H = p.num_heads;
  const int KVH = p.num_kv_heads;
  int kvh, s, part;
  int len_ranked = -1;                // the sequence's length, when the ranking read it
  if constexpr (PART) {
    kvh = blockIdx.x;
    s = blockIdx.y;
    part = blockIdx.z;
  } else {
    const int pos = p.order_by_length
                        ? snake_position((int)blockIdx.x, (int)gridDim.x, p.num_cus)
                        : (int)blockIdx.x;
    const int rank = pos / KVH;
    kvh = pos % KVH;
    s = p.order_by_length
            ? seq_by_rank(p.context_lens, p.num_seqs, BS, rank, s_hist + wave * kSchedKeys, lane,
                          len_ranked)
            : rank;
    part = 0;
  }
  const int G = H / KVH;
  const int L = (!PART && p.order_by_length) ? len_ranked : p.context_lens[s];
  const int MB = p.max_blocks_per_seq;

  const int tiles_per_part = PART ? p.partition_size / BS : 0;
  const int seq_tiles = (L + BS - 1) / BS;
  const int tile0 = PART ? part * tiles_per_part : 0;
  if (PART && L > 0 && tile0 >= seq_tiles) return;
  const int ntiles_all = PART ? min(seq_tiles - tile0, tiles_per_part) : seq_tiles;
  const int share = (ntiles_all + WAVES - 1) / WAVES;
  const int my_first = tile0 + wave * share;          // first tile of this wavefront
  const int ntiles = max(0, min(share, ntiles_all - wave * share));
  const int last_tile = tile0 + ntiles_all - 1;       // the only tile that can be partial
  const bool bad_len = (L < 0) || (L > MB * BS);
  const bool head_ok = n < G;
  const int h = kvh * G + n;
  const int64_t prow = (int64_t)(s * H + h) * (PART ? p.num_partitions : 1) + part;

  // Output row m of product j is head dim 16E(j/E) + E m + j%E, so lane (n, g)
  // holds, for each i, the 4E consecutive dims starting at 16E i + 4E g:
  // dim offset E r + e comes from product E i + e, row 4g + r.
  auto write_out = [&](const float4_t (&o)[NPV]) {
    if (!head_ok) return;
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      float run[4 * E];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) run[E * r + e] = o[E * i + e][r];
      const int d0 = 16 * E * i + 4 * E * g;
      if constexpr (PART) {
#pragma unroll
        for (int c = 0; c < E; ++c)
          *reinterpret_cast<float4_t*>(p.tmp_out + prow * D + d0 + 4 * c) =
              float4_t{run[4 * c], run[4 * c + 1], run[4 * c + 2], run[4 * c + 3]};
      } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + (int64_t)(s * H + h) * D + d0;
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
    }
  };

  // The step's new token (fused append) goes to the last wavefront, whose
  // share of tiles is the smallest: it stores the token in its slot (which
  // no workgroup of this launch reads unmasked: position L of its sequence
  // is past the context) and takes it as its first token.
  const bool take_new = !PART && p.append != 0 && wave == WAVES - 1;
  NewToken<D> nt;
  int32_t slot = -1;
  if (take_new) slot = p.slot_mapping[s];

  if (bad_len || (PART && L <= 0)) {
    if (take_new) {
      nt.load(p, s, kvh, lane);
      nt.template stage<QT, CT>(p, lane, s_new, s_new_bits);
      NewToken<D>::template write<CT, BS>(p, slot, kvh, lane, s_new_bits);
    }
    if (bad_len && wave == 0) {
      float4_t o[NPV];
      const float nanv = __builtin_nanf("");
#pragma unroll
      for (int j = 0; j < NPV; ++j) o[j] = float4_t{nanv, nanv, nanv, nanv};
      write_out(o);
      if (PART && head_ok && g == 0) {
        p.max_logits[prow] = nanv;
        p.exp_sums[prow] = nanv;
      }
    }
    return;
  }

  // Q^T operand: head n of the group, dims in the QK chunk order
  u32x4_t qb[NQK];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       ((int64_t)s * p.q_seq_stride + (int64_t)h * D) * 2;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      qb[c] = head_ok ? *reinterpret_cast<const u32x4_t*>(qrow + qk_dim<ESZ>(c, g) * 2)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE_BYTES;
  const int64_t block_stride = (int64_t)KVH * TILE_BYTES;
  TableSlice tw;
  tw.init(p.block_table + (int64_t)s * MB + my_first, ntiles, p.num_blocks, lane,
          s_table + wave * kWave);

  // per-lane byte offsets inside a tile
  uint32_t koff[SUB][NKL];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int i = 0; i < NKL; ++i)
      koff[u][i] = (uint32_t)((16 * u + n) * D * ESZ +
                              (ESZ == 2 ? qk_dim<2>(i, g) * 2 : 64 * i + 16 * g));
  // V tile [BS/4][D][4]: lane (n, g) reads, for load i of sub-tile u, the 16
  // bytes of token quad 4u + g at head dims E(16 i + n) .. E(16 i + n) + E - 1
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
      for (int i = 0; i < NKL; ++i) kd[u][i] = stream_load16(rk, koff[u][i]);
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int i = 0; i < NVL; ++i) vd[u][i] = stream_load16(rv, voff[u][i]);
  };

  // Softmax state of head n, base 2.  m is the reference the weights are
  // taken against, the same in all four lane groups; it only moves when a
  // logit exceeds it by more than kSlack (so weights stay <= 2^kSlack and
  // most sub-tiles skip the cross-group max and the rescale).  mx is this
  // lane's true running max.
  constexpr float kSlack = 8.0f;
  float m = kNegInf;
  float mx = kNegInf;
  float l = 0.0f;         // partial sum over this lane group's tokens
  float4_t acc[NPV];
#pragma unroll
  for (int j = 0; j < NPV; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int last_len = L - last_tile * BS;

  // K chunk c of a sub-tile as the 16-bit A operand
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
  // A operand of product j = E i + e: head dim row E(16 i + n) + e, tokens
  // 4g .. 4g+3 of the sub-tile, as four 16-bit values
  auto v_operand = [&](const u32x4_t& w, int e) -> u32x2_t {
    if constexpr (ESZ == 2) {
      return u32x2_t{w[2 * e], w[2 * e + 1]};
    } else {
      const uint32_t v = w[e];
      return u32x2_t{MV::template fp8x2<false>(v), MV::template fp8x2<true>(v)};
    }
  };

  auto process = [&](const u32x4_t (&kd)[SUB][NKL], const u32x4_t (&vd)[SUB][NVL], bool masked) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      float4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NQK; ++c) sc = M::qk(k_operand(kd[u], c), qb[c], sc);
      float x[4];
      bool ok[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = sc[r] * p.qk_scale_log2;
        ok[r] = !masked || (16 * u + 4 * g + r) < last_len;
        x[r] = ok[r] ? x[r] : kNegInf;
      }
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, mt);
      if (__builtin_amdgcn_ballot_w64(mt > m + kSlack) != 0) {
        // raise each head's reference to the larger of it and this
        // sub-tile's max (earlier logits stay within kSlack of it)
        mt = xor_max<32>(xor_max<16>(mt));
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
        // residuals are exact in fp32; hi + lo carries 16 bits of each weight
        pl = u32x2_t{MV::pack(pr[0] - MV::lo(p01), pr[1] - MV::hi(p01)),
                     MV::pack(pr[2] - MV::lo(p23), pr[3] - MV::hi(p23))};
        l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      } else {
        // the sum adds the rounded weights the product uses
        l += (MV::lo(p01) + MV::hi(p01)) + (MV::lo(p23) + MV::hi(p23));
      }
      const u32x2_t pb = {p01, p23};
      uint32_t keep0 = 0xFFFFFFFFu, keep1 = 0xFFFFFFFFu;
      if (masked) {
        keep0 = (ok[0] ? 0x0000FFFFu : 0u) | (ok[1] ? 0xFFFF0000u : 0u);
        keep1 = (ok[2] ? 0x0000FFFFu : 0u) | (ok[3] ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        u32x2_t a = v_operand(vd[u][j / E], j % E);
        if (masked) a = u32x2_t{a[0] & keep0, a[1] & keep1};
        acc[j] = MV::pv(a, pb, acc[j]);
      }
      if constexpr (kSplitP) {
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
          u32x2_t a = v_operand(vd[u][j / E], j % E);
          if (masked) a = u32x2_t{a[0] & keep0, a[1] & keep1};
          acc[j] = MV::pv(a, pl, acc[j]);
        }
      }
    }
  };

  // the new token's loads go first, then the prologue's tile loads
  if (take_new) nt.load(p, s, kvh, lane);
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(kb[u], vb[u], u);

  if (take_new) {
    // the token's cached values land in s_new (its store into the cache
    // comes after the stream).  Logit: lane group g's q dims (qb) against
    // the same dims of the cached K row
    nt.template stage<QT, CT>(p, lane, s_new, s_new_bits);
    __builtin_amdgcn_wave_barrier();
    float xn = 0.0f;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      const float4_t k0 = *reinterpret_cast<const float4_t*>(s_new + qk_dim<ESZ>(c, g));
      const float4_t k1 = *reinterpret_cast<const float4_t*>(s_new + qk_dim<ESZ>(c, g) + 4);
      const float kk[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xn = fmaf(M::lo(qb[c][w]), kk[2 * w], xn);
        xn = fmaf(M::hi(qb[c][w]), kk[2 * w + 1], xn);
      }
    }
    xn = xor_add<32>(xor_add<16>(xn));
    m = xn * p.qk_scale_log2;            // reference = its logit: weight 1
    mx = m;
    l = (g == 0) ? 1.0f : 0.0f;          // the four lane groups' sums add up
    // its V row starts the accumulators: element E r + e of run i is
    // output dim 16E i + 4E g + E r + e
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      float run[4 * E];
#pragma unroll
      for (int c = 0; c < E; ++c) {
        const float4_t v4 =
            *reinterpret_cast<const float4_t*>(s_new + D + 16 * E * i + 4 * E * g + 4 * c);
        run[4 * c] = v4[0];
        run[4 * c + 1] = v4[1];
        run[4 * c + 2] = v4[2];
        run[4 * c + 3] = v4[3];
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[E * i + e][r] = run[E * r + e];
    }
  }

  for (int t0 = 0; t0 < ntiles; t0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int t = t0 + u;
      issue(kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF], t + NBUF - 1);
      if (t < ntiles) process(kb[u], vb[u], (my_first + t == last_tile) && (last_len < BS));
    }
  }

  // the new token into its slot, after the stream
  if (take_new) NewToken<D>::template write<CT, BS>(p, slot, kvh, lane, s_new_bits);

  bool bad = table_bad(tw);
  if constexpr (WAVES > 1) {
    // merge the wavefronts' states (each with its own reference max)
    if (wave > 0) {
      float* st = s_state + ((wave - 1) * kWave + lane) * NSTATE;
#pragma unroll
      for (int j = 0; j < NPV; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[4 * j + r] = acc[j][r];
      st[NPV * 4 + 0] = m;
      st[NPV * 4 + 1] = mx;
      st[NPV * 4 + 2] = l;
      st[NPV * 4 + 3] = bad ? 1.0f : 0.0f;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float* st = s_state + ((w - 1) * kWave + lane) * NSTATE;
      const float mo = st[NPV * 4 + 0];
      const float mn = fmaxf(m, mo);
      const float fa = (m == mn) ? 1.0f : exp2_hw(m - mn);
      const float fb = (mo == mn) ? 1.0f : exp2_hw(mo - mn);
#pragma unroll
      for (int j = 0; j < NPV; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = acc[j][r] * fa + st[4 * j + r] * fb;
      l = l * fa + st[NPV * 4 + 2] * fb;
      mx = fmaxf(mx, st[NPV * 4 + 1]);
      bad |= st[NPV * 4 + 3] != 0.0f;
      m = mn;
    }
  }

  // the normaliser of head n: sum over the four lane groups; the partial
  // triple reports the exact max, with the sum re-referenced to it
  l = xor_add<32>(xor_add<16>(l));
  mx = xor_max<32>(xor_max<16>(mx));

  float4_t o[NPV];
  const float nanv = __builtin_nanf("");
  const bool empty = ntiles_all <= 0 && (PART || p.append == 0);
  // one division per lane; empty contexts give 0, bad ones NaN
  const float inv = bad ? nanv : (empty ? 0.0f : p.v_scale / l);
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) o[j][r] = acc[j][r] * inv;   // NaN when bad
  }
  write_out(o);
  if constexpr (PART) {
    if (head_ok && g == 0) {
      p.max_logits[prow] = bad ? nanv : mx * kLn2;
      p.exp_sums[prow] = bad ? nanv : (mx == m ? l : l * exp2_hw(m - mx));
    }
  }
}

template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid = PART ? dim3(p.num_kv_heads, p.num_seqs, p.num_partitions)
                        : dim3(p.num_kv_heads * p.num_seqs, 1, 1);
  hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, D, BS, PART, WAVES>), grid, dim3(64 * WAVES), 0,
                     stream, p);
  return hipGetLastError();
}

// Partitions already give every wavefront a bounded share: one wavefront per
// workgroup.  One pass: PA_MFMA_WAVES wavefronts split each sequence.
template <typename QT, typename CT, int D, int BS>
hipError_t pick_part(const DecodeParams& p, bool part, hipStream_t st) {
  return part ? launch_one<QT, CT, D, BS, true, 1>(p, st)
              : launch_one<QT, CT, D, BS, false, PA_MFMA_WAVES>(p, st);
}
template <typename QT, typename CT, int D>
hipError_t pick_bs(const DecodeParams& p, int bs, bool part, hipStream_t st) {
  return bs == 16 ? pick_part<QT, CT, D, 16>(p, part, st) : pick_part<QT, CT, D, 32>(p, part, st);
}
template <typename QT, typename CT>
hipError_t pick_d(const DecodeParams& p, int d, int bs, bool part, hipStream_t st) {
  return d == 64 ? pick_bs<QT, CT, 64>(p, bs, part, st) : pick_bs<QT, CT, 128>(p, bs, part, st);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, Dt q_dt, Dt cache_dt, int head_size,
                              int block_size, bool partitioned, hipStream_t stream) {
  if (q_dt == Dt::F16) {
    return cache_dt == Dt::FP8 ? pick_d<F16, FP8>(p, head_size, block_size, partitioned, stream)
                               : pick_d<F16, F16>(p, head_size, block_size, partitioned, stream);
  }
  return cache_dt == Dt::FP8 ? pick_d<BF16, FP8>(p, head_size, block_size, partitioned, stream)
                             : pick_d<BF16, BF16>(p, head_size, block_size, partitioned, stream);
}

}  // namespace pa
