// Paged decode attention, one query head per kv head (num_heads == num_kv_heads),
// on the vector ALUs of gfx950.
//
// Method (vLLM "Paged Attention" design page, sections "QK", "Softmax",
// "Value", "LV", "Output"): for one (sequence, head[, partition]) the kernel
// reads every K/V tile of the context through the block table, takes the
// scaled dot products with q, a numerically stable softmax and the weighted
// sum of V.  The design page's CUDA kernel is prior art only; this kernel is
// laid out for 64-lane wavefronts:
//
//  * A workgroup of WAVES wavefronts takes one (sequence, head[, partition]);
//    wavefront w streams the w-th contiguous share of its tiles and the
//    states merge in LDS at the end.
//  * A (block, kv head) tile is contiguous in HBM: K [BS][D] token-major and
//    V [BS/4][D][4] (each group of four tokens holds the D head dims, each
//    with the four tokens' values).  Each lane issues 16-byte raw buffer loads
//    at lane*16 + i*1024, so every load instruction moves one contiguous KiB.
//    The tile's descriptor base is the tile address; a zero-length descriptor
//    turns prefetches past the end of the range into free zero fills, so the
//    prefetch pipeline (NBUF tiles in flight) needs no branches.
//  * QK: a lane holds VEC consecutive dims of one token; D/VEC lanes reduce
//    the dot product with DPP row operations.
//  * Softmax is online with one reference max per wavefront (base 2: scores
//    are pre-multiplied by scale * log2(e) and 2^x is v_exp_f32).  The
//    reference only moves when a logit exceeds it by more than 2^8 (a ballot
//    decides, then one wave-wide max and a rescale), so the usual tile costs
//    one exponential per token and no cross-lane traffic besides LDS.
//  * The weights of a tile go through LDS to the V lanes: a V lane owns E
//    whole head dims (E = 2 for 16-bit, 4 for fp8 caches) over its token
//    quads, so partial outputs of lanes that share dims just add at the end.
//  * Tokens past the context (last, partial tile only) get weight 0 and
//    their V values are skipped by selects, never multiplied by zero, so
//    stale or NaN slots have no influence.
//  * The block table comes through the shared TableWindow (64 entries per
//    VGPR, v_readlane per tile); bad entries give a NaN row, never a read.
#include "pa_decode_common.h"
#include "pa_kernels.h"

#ifndef PA_VALU_NBUF
#define PA_VALU_NBUF 3
#endif
#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 4
#endif

namespace pa {
namespace {

template <typename CT, int D>
struct QFrag;

// 16-bit cache: q kept packed (8 elements, 16 bytes) for v_dot2.
template <int D>
struct QFrag<F16, D> {
  u32x4_t w;
};
template <int D>
struct QFrag<BF16, D> {
  u32x4_t w;
};
// fp8 cache: q as 16 fp32 values.
template <int D>
struct QFrag<FP8, D> {
  float f[16];
};

template <typename QT, typename CT, int D>
__device__ __forceinline__ QFrag<CT, D> load_q(const void* qrow, int c) {
  QFrag<CT, D> fr;
  if constexpr (CT::kBytes == 2) {
    fr.w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(qrow) + c * 16);
  } else {
    const u32x4_t* src =
        reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(qrow) + c * 32);
    u32x4_t a = src[0], b = src[1];
    uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (__is_same(QT, F16)) {
        fr.f[2 * i] = f16_lo(w[i]);
        fr.f[2 * i + 1] = f16_hi(w[i]);
      } else {
        fr.f[2 * i] = bf16_lo(w[i]);
        fr.f[2 * i + 1] = bf16_hi(w[i]);
      }
    }
  }
  return fr;
}

// Partial dot product of one 16-byte K chunk with the lane's q fragment.
template <typename CT, int D>
__device__ __forceinline__ float dot_chunk(const QFrag<CT, D>& q, u32x4_t k) {
  if constexpr (__is_same(CT, F16)) {
    float a = __builtin_amdgcn_fdot2(as_half2(q.w[0]), as_half2(k[0]), 0.0f, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[1]), as_half2(k[1]), a, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[2]), as_half2(k[2]), a, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[3]), as_half2(k[3]), a, false);
    return a;
  } else if constexpr (__is_same(CT, BF16)) {
    float a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[0]), as_bf162(k[0]), 0.0f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[1]), as_bf162(k[1]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[2]), as_bf162(k[2]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[3]), as_bf162(k[3]), a, false);
    return a;
  } else {
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float2_t lo = fp8x2_to_f32<false>(k[w]);
      float2_t hi = fp8x2_to_f32<true>(k[w]);
      a = fmaf(q.f[4 * w + 0], lo[0], a);
      a = fmaf(q.f[4 * w + 1], lo[1], a);
      a = fmaf(q.f[4 * w + 2], hi[0], a);
      a = fmaf(q.f[4 * w + 3], hi[1], a);
    }
    return a;
  }
}

// The E x 4 values of one 16-byte V chunk (E head dims, 4 tokens each), fp32:
// out[e][r] = dim e of the chunk, token r of the quad.
template <typename CT, int E>
__device__ __forceinline__ void v_chunk(const u32x4_t& w, float (&out)[E][4]) {
  if constexpr (CT::kBytes == 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float2_t lo = fp8x2_to_f32<false>(w[e]);
      const float2_t hi = fp8x2_to_f32<true>(w[e]);
      out[e][0] = lo[0];
      out[e][1] = lo[1];
      out[e][2] = hi[0];
      out[e][3] = hi[1];
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t a = w[2 * e], b = w[2 * e + 1];
      if constexpr (__is_same(CT, F16)) {
        out[e][0] = f16_lo(a);
        out[e][1] = f16_hi(a);
        out[e][2] = f16_lo(b);
        out[e][3] = f16_hi(b);
      } else {
        out[e][0] = bf16_lo(a);
        out[e][1] = bf16_hi(a);
        out[e][2] = bf16_lo(b);
        out[e][3] = bf16_hi(b);
      }
    }
  }
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kSlack = 8.0f;   // weights stay <= 2^8 between reference moves

template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_valu_kernel(const DecodeParams p) {
  constexpr int ESZ = CT::kBytes;
  constexpr int VEC = 16 / ESZ;             // cache elements per 16-byte lane load
  constexpr int TILE_BYTES = BS * D * ESZ;  // one (block, kv head) tile of K or of V
  constexpr int NLOAD = TILE_BYTES / 1024;  // 16-byte loads per lane per tile
  constexpr int LPT = D / VEC;              // K: lanes per token
  constexpr int TPI = kWave / LPT;          // K: tokens per load instruction
  constexpr int E = 16 / (4 * ESZ);         // V: head dims per 16-byte chunk
  constexpr int LPQ = D / E;                // V: lanes per token quad
  constexpr int QPI = kWave / LPQ;          // V: token quads per load instruction
  constexpr int NBUF = PA_VALU_NBUF;
  static_assert(NLOAD * TPI == BS && NLOAD * QPI * 4 == BS, "tile mapping");
  static_assert(LPT >= 1 && LPT <= 16 && NLOAD <= LPT && LPQ <= kWave, "lane mapping");

  constexpr int NSTATE = E + 2;
  __shared__ __attribute__((aligned(16))) float s_p_all[WAVES * BS];
  __shared__ int s_hist[PART ? 1 : WAVES * kSchedKeys];
  __shared__ float s_state[WAVES > 1 ? (WAVES - 1) * kWave * NSTATE : 1];
  __shared__ __attribute__((aligned(16))) float s_new[PART ? 4 : 2 * D];   // fused append
  __shared__ uint16_t s_new_bits[PART ? 2 : 2 * D];
  __shared__ int s_table[table_lds_ints(WAVES)];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int lane = threadIdx.x & 63;
  float* s_p = s_p_all + wave * BS;
  const int H = p.num_heads;
  int h, s, part;
  int len_ranked = -1;                // the sequence's length, when the ranking read it
  if constexpr (PART) {
    if (p.die_order) {
      // partitions: (head, sequence, partition) in partition-major order, the
      // positions spread over the dies like those of a one pass
      const int items = H * p.num_seqs * p.num_partitions;
      const int pos = die_position((int)blockIdx.x, (int)gridDim.x / kDies);
      if (pos >= items) return;                         // a spare workgroup
      h = pos % H;
      s = (pos / H) % p.num_seqs;
      part = pos / (H * p.num_seqs);
    } else {
      h = blockIdx.x;
      s = blockIdx.y;
      part = blockIdx.z;
    }
  } else {
    // one pass: workgroup b takes head pos % H of the sequence at position
    // pos / H of the longest-first order, spread over the dies by their
    // streaming rates (or of index order)
    const int pos = p.order_by_length ? die_position((int)blockIdx.x, (int)gridDim.x / kDies)
                                      : (int)blockIdx.x;
    if (pos >= p.num_seqs * H) return;                  // a spare workgroup
    const int rank = pos / H;
    h = pos % H;
    s = p.order_by_length
            ? seq_by_rank(p.context_lens, p.num_seqs, BS, rank, s_hist + wave * kSchedKeys, lane,
                          len_ranked)
            : rank;
    part = 0;
  }
  const int L = (!PART && p.order_by_length) ? len_ranked : p.context_lens[s];
  const int MB = p.max_blocks_per_seq;

  // token range of this workgroup and of this wavefront
  const int tiles_per_part = PART ? p.partition_size / BS : 0;
  const int seq_tiles = (L + BS - 1) / BS;
  const int tile0 = PART ? part * tiles_per_part : 0;
  if (PART && L > 0 && tile0 >= seq_tiles) return;
  const int ntiles_all = PART ? min(seq_tiles - tile0, tiles_per_part) : seq_tiles;
  const int share = (ntiles_all + WAVES - 1) / WAVES;
  const int my_first = tile0 + wave * share;
  const int ntiles = max(0, min(share, ntiles_all - wave * share));
  const int last_tile = tile0 + ntiles_all - 1;       // the only tile that can be partial
  const bool bad_len = (L < 0) || (L > MB * BS);

  const int row = s * H + h;
  const int64_t pidx = (int64_t)row * (PART ? p.num_partitions : 1) + part;

  // lanes l < LPQ own head dims E*l .. E*l + E - 1 of the result
  auto write_row = [&](const float (&vals)[E]) {
    if (lane >= LPQ) return;
    if constexpr (PART) {
      float* dst = p.tmp_out + pidx * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = vals[e];
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + (int64_t)row * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        *reinterpret_cast<uint32_t*>(dst + e) =
            (uint32_t)to_bits16<QT>(vals[e]) | ((uint32_t)to_bits16<QT>(vals[e + 1]) << 16);
      }
    }
  };

  // query head h reads kv head h / G (contiguous groups); this kernel is the
  // one-head-per-kv-head path, but stays correct for any G
  const int G = H / p.num_kv_heads;
  const int kvh = h / G;
  // The step's new token (fused append) goes to the last wavefront, whose
  // share of tiles is the smallest: it takes the token as its first one,
  // and (one query head per kv head doing it) stores it in its slot, which
  // no workgroup of this launch reads unmasked (position L of its sequence
  // is past the context).
  const bool take_new = !PART && p.append != 0 && wave == WAVES - 1;
  NewToken<D> nt;
  int32_t slot = -1;
  if (take_new) slot = h % G == 0 ? p.slot_mapping[s] : -1;

  if (bad_len || (PART && L <= 0)) {
    if (take_new) {
      nt.load(p, s, kvh, lane);
      nt.template stage<QT, CT>(p, lane, s_new, s_new_bits);
      NewToken<D>::template write<CT, BS>(p, slot, kvh, lane, s_new_bits);
    }
    if (bad_len && wave == 0) {
      float nanv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) nanv[e] = __builtin_nanf("");
      write_row(nanv);
      if (PART && lane == 0) {
        p.max_logits[pidx] = __builtin_nanf("");
        p.exp_sums[pidx] = __builtin_nanf("");
      }
    }
    return;   // partitioned with an empty context: nothing to write
  }

  const char* qrow = reinterpret_cast<const char*>(p.q) +
                     ((int64_t)s * p.q_seq_stride + (int64_t)h * D) * sizeof(uint16_t);
  const QFrag<CT, D> qf = load_q<QT, CT, D>(qrow, lane % LPT);

  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE_BYTES;
  const int64_t block_stride = (int64_t)p.num_kv_heads * TILE_BYTES;
  TableSlice tw;
  tw.init(p.block_table + (int64_t)s * MB + my_first, ntiles, p.num_blocks, lane,
          s_table + wave * kWave);

  u32x4_t kb[NBUF][NLOAD];
  u32x4_t vb[NBUF][NLOAD];

  auto issue = [&](u32x4_t (&kd)[NLOAD], u32x4_t (&vd)[NLOAD], int n) {
    int phys = 0;
    uint32_t bytes = 0;
    if (n < ntiles) {
      phys = tw.phys(n, lane);
      bytes = TILE_BYTES;
    }
    const int64_t off = (int64_t)phys * block_stride;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) kd[i] = stream_load16(rk, lane * 16 + i * 1024);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) vd[i] = stream_load16(rv, lane * 16 + i * 1024);
  };

  float m = kNegInf;       // reference max of this wavefront (wave-uniform)
  float mx = kNegInf;      // exact running max of this lane's logits
  float l = 0.0f;          // sum of this lane's token weights (its K token row)
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;

  const int c_k = lane % LPT;           // K: chunk of the token's dims
  const int tok_k = lane / LPT;         // K: token within an instruction
  const int quad_v = lane / LPQ;        // V: token quad within an instruction
  const int last_len = L - last_tile * BS;

  auto process = [&](const u32x4_t (&kd)[NLOAD], const u32x4_t (&vd)[NLOAD], bool masked) {
    // logits of tokens i*TPI + tok_k
    float x[NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      x[i] = group_sum<LPT>(dot_chunk<CT, D>(qf, kd[i])) * p.qk_scale_log2;
      if (masked) x[i] = (i * TPI + tok_k) < last_len ? x[i] : kNegInf;
    }
    float mt = x[0];
#pragma unroll
    for (int i = 1; i < NLOAD; ++i) mt = fmaxf(mt, x[i]);
    mx = fmaxf(mx, mt);
    if (__builtin_amdgcn_ballot_w64(mt > m + kSlack) != 0) {
      const float mn = fmaxf(m, wave_max(mt));
      const float alpha = (m == mn) ? 1.0f : exp2_hw(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= alpha;
    }
    float pw[NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      pw[i] = exp2_hw(x[i] - m);        // masked: 2^-inf = 0
      l += pw[i];
    }
    float mine = pw[0];
#pragma unroll
    for (int i = 1; i < NLOAD; ++i) mine = (c_k == i) ? pw[i] : mine;
    __builtin_amdgcn_wave_barrier();
    if (c_k < NLOAD) s_p[c_k * TPI + tok_k] = mine;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int q = i * QPI + quad_v;                       // token quad of chunk i
      const float4_t w4 = *reinterpret_cast<const float4_t*>(&s_p[4 * q]);
      float v[E][4];
      v_chunk<CT, E>(vd[i], v);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = !masked || (4 * q + r) < last_len;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = ok ? fmaf(w4[r], v[e][r], acc[e]) : acc[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // the new token's loads go first, then the prologue: NBUF - 1 tiles in
  // flight
  if (take_new) nt.load(p, s, kvh, lane);
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(kb[u], vb[u], u);

  if (take_new) {
    // the token's cached values land in s_new (its store into the cache
    // comes after the stream).  Logit: the lane's q chunk against the same
    // dims of the cached K row, summed over the LPT lanes of a row
    nt.template stage<QT, CT>(p, lane, s_new, s_new_bits);
    __builtin_amdgcn_wave_barrier();
    const float* kk = s_new + (lane % LPT) * VEC;
    float xp = 0.0f;
    if constexpr (CT::kBytes == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float2_t k2 = *reinterpret_cast<const float2_t*>(kk + 2 * w);
        xp = fmaf(in_lo<QT>(qf.w[w]), k2[0], xp);
        xp = fmaf(in_hi<QT>(qf.w[w]), k2[1], xp);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const float4_t k4 = *reinterpret_cast<const float4_t*>(kk + j);
        xp = fmaf(qf.f[j], k4[0], xp);
        xp = fmaf(qf.f[j + 1], k4[1], xp);
        xp = fmaf(qf.f[j + 2], k4[2], xp);
        xp = fmaf(qf.f[j + 3], k4[3], xp);
      }
    }
    m = group_sum<LPT>(xp) * p.qk_scale_log2;   // reference = its logit: weight 1
    mx = m;
    if (lane < LPT) l = 1.0f;            // one K token row counts it
    if (lane < LPQ) {                    // one token quad row adds its V
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = s_new[D + E * lane + e];
    }
  }

  for (int n0 = 0; n0 < ntiles; n0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int n = n0 + u;
      issue(kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF], n + NBUF - 1);
      if (n < ntiles) {
        const bool masked = (my_first + n == last_tile) && (last_len < BS);
        process(kb[u], vb[u], masked);
      }
    }
  }

  // the new token into its slot (slot -1: another head of the group stores
  // it), after the stream
  if (take_new) NewToken<D>::template write<CT, BS>(p, slot, kvh, lane, s_new_bits);

  // lanes sharing head dims add up (one reference max); the weight sum adds
  // one lane per K token row
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = sum_lanes_mod<LPQ>(acc[e]);
  l = sum_lanes_mod<LPT>(l);

  bool bad = table_bad(tw);
  if constexpr (WAVES > 1) {
    // merge the wavefronts' states (lane i holds the same dims in every one)
    if (wave > 0) {
      float* st = s_state + ((wave - 1) * kWave + lane) * NSTATE;
#pragma unroll
      for (int e = 0; e < E; ++e) st[e] = acc[e];
      st[E] = m;
      st[E + 1] = bad ? -l - 1.0f : l;   // sign marks a bad table entry
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float* st = s_state + ((w - 1) * kWave + lane) * NSTATE;
      const float mo = st[E];
      float lo = st[E + 1];
      if (lo < 0.0f) {
        bad = true;
        lo = -lo - 1.0f;
      }
      const float mn = fmaxf(m, mo);
      const float fa = (m == mn) ? 1.0f : exp2_hw(m - mn);
      const float fb = (mo == mn) ? 1.0f : exp2_hw(mo - mn);
      l = l * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = acc[e] * fa + st[e] * fb;
      m = mn;
    }
  }

  float res[E];
  const bool empty = ntiles_all <= 0 && (PART || p.append == 0);
  const float inv = bad ? __builtin_nanf("") : (empty ? 0.0f : p.v_scale / l);
#pragma unroll
  for (int e = 0; e < E; ++e) res[e] = acc[e] * inv;   // NaN when bad
  write_row(res);
  if constexpr (PART) {
    // the partial triple reports the exact max, with the sum re-referenced
    const float mw = wave_max(mx);
    if (lane == 0) {
      p.max_logits[pidx] = bad ? __builtin_nanf("") : mw * kLn2;
      p.exp_sums[pidx] = bad ? __builtin_nanf("") : (mw == m ? l : l * exp2_hw(m - mw));
    }
  }
}

// Launches take the die order up to kDieMaxItems items (the positions'
// virtual times stay within 32 bits); beyond that, partitions take the plain
// 3-D grid and a one pass the index order.
#ifndef PA_DIE_MAX_ITEMS
#define PA_DIE_MAX_ITEMS (int64_t(1) << 27)
#endif
constexpr int64_t kDieMaxItems = PA_DIE_MAX_ITEMS;

template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
hipError_t launch_one(const DecodeParams& params, hipStream_t stream) {
  DecodeParams p = params;
  const int64_t part_items = (int64_t)p.num_heads * p.num_seqs * p.num_partitions;
  p.die_order = PART && part_items <= kDieMaxItems ? 1 : 0;
  if (!PART && (int64_t)p.num_heads * p.num_seqs > kDieMaxItems) p.order_by_length = 0;
  const dim3 grid = PART ? (p.die_order ? dim3(kDies * die_workgroups((int)part_items), 1, 1)
                                        : dim3(p.num_heads, p.num_seqs, p.num_partitions))
                        : dim3(p.order_by_length ? kDies * die_workgroups(p.num_heads * p.num_seqs)
                                                 : p.num_heads * p.num_seqs,
                               1, 1);
  hipLaunchKernelGGL((decode_valu_kernel<QT, CT, D, BS, PART, WAVES>), grid, dim3(64 * WAVES), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename QT, typename CT, int D, int BS>
hipError_t pick_part(const DecodeParams& p, bool part, hipStream_t st) {
  return part ? launch_one<QT, CT, D, BS, true, 1>(p, st)
              : launch_one<QT, CT, D, BS, false, PA_VALU_WAVES>(p, st);
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

hipError_t launch_decode_valu(const DecodeParams& p, Dt q_dt, Dt cache_dt, int head_size,
                              int block_size, bool partitioned, hipStream_t stream) {
  if (q_dt == Dt::F16) {
    return cache_dt == Dt::FP8 ? pick_d<F16, FP8>(p, head_size, block_size, partitioned, stream)
                               : pick_d<F16, F16>(p, head_size, block_size, partitioned, stream);
  }
  return cache_dt == Dt::FP8 ? pick_d<BF16, FP8>(p, head_size, block_size, partitioned, stream)
                             : pick_d<BF16, BF16>(p, head_size, block_size, partitioned, stream);
}

}  // namespace pa
