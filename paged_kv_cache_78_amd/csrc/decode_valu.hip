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
//  * One wavefront = one workgroup = one (sequence, head[, partition]).
//  * A (block, kv head) tile is contiguous in HBM: K [BS][D] token-major and
//    V [D][BS] dim-major.  Each lane issues 16-byte raw buffer loads at
//    lane*16 + i*1024, so every load instruction moves one contiguous KiB.
//    The tile's descriptor base is the tile address; a zero-length descriptor
//    turns prefetches past the end of the range into free zero fills, so the
//    prefetch pipeline (NBUF tiles in flight) needs no branches.
//  * QK: a lane holds VEC consecutive dims of one token; D/VEC lanes reduce
//    the dot product with DPP row operations.
//  * The scores go through 64-256 bytes of LDS to the lanes that hold the
//    matching V columns: a V lane owns NLOAD rows (head dims) over VEC tokens.
//  * Softmax is online and private to each lane (running max m, sum l and
//    the NLOAD partial outputs, in base 2: scores are pre-multiplied by
//    scale * log2(e) and 2^x is the hardware v_exp_f32).  The lanes that
//    share a row merge (m, l, acc) once at the end, with DPP.
//  * Tokens past the context (last, partial tile only) are excluded by
//    selects, never by multiplying with zero, so stale or NaN slots have no
//    influence.
//  * The block-table slice is read 64 entries at a time into one VGPR and
//    broadcast per tile with v_readlane; the next 64 are loaded a chunk ahead.
//    Ids outside [0, num_blocks) are replaced by 0 before any address is
//    formed and make the row NaN.
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
    float a = __builtin_amdgcn_fdot2(as_half2(q.w[0]),
                                     as_half2(k[0]), 0.0f, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[1]),
                               as_half2(k[1]), a, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[2]),
                               as_half2(k[2]), a, false);
    a = __builtin_amdgcn_fdot2(as_half2(q.w[3]),
                               as_half2(k[3]), a, false);
    return a;
  } else if constexpr (__is_same(CT, BF16)) {
    float a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[0]),
                                              as_bf162(k[0]), 0.0f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[1]),
                                        as_bf162(k[1]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[2]),
                                        as_bf162(k[2]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q.w[3]),
                                        as_bf162(k[3]), a, false);
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

// Element j of a 16-byte V chunk as fp32.
template <typename CT>
__device__ __forceinline__ float v_elem(const u32x4_t& v, int j) {
  if constexpr (__is_same(CT, F16)) {
    return (j & 1) ? f16_hi(v[j >> 1]) : f16_lo(v[j >> 1]);
  } else if constexpr (__is_same(CT, BF16)) {
    return (j & 1) ? bf16_hi(v[j >> 1]) : bf16_lo(v[j >> 1]);
  } else {
    float2_t pr = ((j >> 1) & 1) ? fp8x2_to_f32<true>(v[j >> 2]) : fp8x2_to_f32<false>(v[j >> 2]);
    return pr[j & 1];
  }
}

template <typename CT>
__device__ __forceinline__ void v_decode(const u32x4_t& v, float (&out)[16 / CT::kBytes]) {
  constexpr int VEC = 16 / CT::kBytes;
  if constexpr (CT::kBytes == 1) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float2_t lo = fp8x2_to_f32<false>(v[w]);
      float2_t hi = fp8x2_to_f32<true>(v[w]);
      out[4 * w + 0] = lo[0];
      out[4 * w + 1] = lo[1];
      out[4 * w + 2] = hi[0];
      out[4 * w + 3] = hi[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < VEC; ++j) out[j] = v_elem<CT>(v, j);
  }
}

constexpr float kNegInf = -__builtin_huge_valf();

template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_valu_kernel(const DecodeParams p) {
  constexpr int ESZ = CT::kBytes;
  constexpr int VEC = 16 / ESZ;             // cache elements per 16-byte lane load
  constexpr int TILE_BYTES = BS * D * ESZ;  // one (block, kv head) tile of K or of V
  constexpr int NLOAD = TILE_BYTES / 1024;  // 16-byte loads per lane per tile
  constexpr int LPT = D / VEC;              // K: lanes per token
  constexpr int TPI = kWave / LPT;          // K: tokens per load instruction
  constexpr int LPR = BS / VEC;             // V: lanes per head-dim row
  constexpr int RPI = kWave / LPR;          // V: rows per load instruction
  constexpr int NBUF = PA_VALU_NBUF;        // tiles resident: 1 in use, the rest in flight
  static_assert(NLOAD * TPI == BS && NLOAD * RPI == D, "tile mapping");
  static_assert(LPT >= 1 && LPT <= 16 && LPR >= 1 && LPR <= 4 && NLOAD <= LPT, "lane mapping");

  // WAVES wavefronts share one (sequence, head[, partition]): wavefront w
  // takes the w-th contiguous share of its tiles; the states merge in LDS.
  constexpr int NSTATE = NLOAD + 2;
  __shared__ __attribute__((aligned(16))) float s_scores_all[WAVES * BS];
  __shared__ int s_hist[PART ? 1 : WAVES * kSchedKeys];
  __shared__ float s_state[WAVES > 1 ? (WAVES - 1) * kWave * NSTATE : 1];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float* s_scores = s_scores_all + wave * BS;
  const int H = p.num_heads;
  int h, s, part;
  if constexpr (PART) {
    h = blockIdx.x;
    s = blockIdx.y;
    part = blockIdx.z;
  } else {
    // one pass: workgroup b takes head b % H of the sequence at position
    // b / H of the longest-first order (or of index order)
    const int pos = p.order_by_length
                        ? snake_position((int)blockIdx.x, (int)gridDim.x, p.num_cus)
                        : (int)blockIdx.x;
    const int rank = pos / H;
    h = pos % H;
    s = p.order_by_length
            ? seq_by_rank(p.context_lens, p.num_seqs, BS, rank, s_hist + wave * kSchedKeys, lane)
            : rank;
    part = 0;
  }
  const int L = p.context_lens[s];
  const int MB = p.max_blocks_per_seq;

  // token range of this workgroup
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

  // output row addressing
  const int row = s * H + h;
  float* part_out = PART ? p.tmp_out + ((int64_t)row * p.num_partitions + part) * D : nullptr;

  auto write_row = [&](const float (&vals)[NLOAD], bool valid_lane) {
    if (!valid_lane) return;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int d = i * RPI + lane / LPR;
      if constexpr (PART) {
        part_out[d] = vals[i];
      } else {
        reinterpret_cast<uint16_t*>(p.out)[(int64_t)row * D + d] = to_bits16<QT>(vals[i]);
      }
    }
  };

  if (bad_len || (PART && L <= 0 && !bad_len)) {
    if (bad_len && wave == 0) {
      float nanv[NLOAD];
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) nanv[i] = __builtin_nanf("");
      write_row(nanv, lane % LPR == 0);
      if (PART && lane == 0) {
        p.max_logits[(int64_t)row * p.num_partitions + part] = __builtin_nanf("");
        p.exp_sums[(int64_t)row * p.num_partitions + part] = __builtin_nanf("");
      }
    }
    return;   // partitioned with an empty context: nothing to write
  }

  // query head h reads kv head h / G (contiguous groups); this kernel is the
  // one-head-per-kv-head path, but stays correct for any G
  const int kvh = h / (H / p.num_kv_heads);
  const char* qrow = reinterpret_cast<const char*>(p.q) +
                     ((int64_t)s * p.q_seq_stride + (int64_t)h * D) * sizeof(uint16_t);
  const QFrag<CT, D> qf = load_q<QT, CT, D>(qrow, lane % LPT);

  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE_BYTES;
  const int64_t block_stride = (int64_t)p.num_kv_heads * TILE_BYTES;
  TableWindow tw;
  tw.init(p.block_table + (int64_t)s * MB + my_first, ntiles, p.num_blocks, lane);

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
    for (int i = 0; i < NLOAD; ++i) kd[i] = buffer_load16(rk, lane * 16 + i * 1024);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) vd[i] = buffer_load16(rv, lane * 16 + i * 1024);
  };

  // per-lane online softmax state (base 2)
  float m = kNegInf;
  float l = 0.0f;
  float acc[NLOAD];
#pragma unroll
  for (int i = 0; i < NLOAD; ++i) acc[i] = 0.0f;

  const int c_k = lane % LPT;          // K: chunk of the token's dims
  const int tok_k = lane / LPT;        // K: token within an instruction
  const int tok_v = (lane % LPR) * VEC;  // V: first token of this lane's columns
  const int last_len = L - last_tile * BS;   // valid tokens in the last tile

  auto process = [&](const u32x4_t (&kd)[NLOAD], const u32x4_t (&vd)[NLOAD], bool masked) {
    // scores of tokens i*TPI + tok_k
    float sc[NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      sc[i] = group_sum<LPT>(dot_chunk<CT, D>(qf, kd[i])) * p.qk_scale_log2;
    }
    float mine = sc[0];
#pragma unroll
    for (int i = 1; i < NLOAD; ++i) mine = (c_k == i) ? sc[i] : mine;
    __builtin_amdgcn_wave_barrier();
    if (c_k < NLOAD) s_scores[c_k * TPI + tok_k] = mine;
    __builtin_amdgcn_wave_barrier();
    float x[VEC];
#pragma unroll
    for (int j = 0; j < VEC; j += 4) {
      float4_t t4 = *reinterpret_cast<const float4_t*>(&s_scores[tok_v + j]);
      x[j] = t4[0];
      x[j + 1] = t4[1];
      x[j + 2] = t4[2];
      x[j + 3] = t4[3];
    }
    __builtin_amdgcn_wave_barrier();
    if (!masked) {
      float mt = x[0];
#pragma unroll
      for (int j = 1; j < VEC; ++j) mt = fmaxf(mt, x[j]);
      const float mn = fmaxf(m, mt);
      const float alpha = exp2_hw(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) acc[i] *= alpha;
      float pj[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        pj[j] = exp2_hw(x[j] - mn);
        l += pj[j];
      }
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        float vv[VEC];
        v_decode<CT>(vd[i], vv);
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[i] = fmaf(pj[j], vv[j], acc[i]);
      }
    } else {
      bool ok[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        ok[j] = (tok_v + j) < last_len;
        x[j] = ok[j] ? x[j] : kNegInf;
      }
      float mt = x[0];
#pragma unroll
      for (int j = 1; j < VEC; ++j) mt = fmaxf(mt, x[j]);
      const float mn = fmaxf(m, mt);
      const float alpha = (m == mn) ? 1.0f : exp2_hw(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) acc[i] *= alpha;
      float pj[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        pj[j] = ok[j] ? exp2_hw(x[j] - mn) : 0.0f;
        l += pj[j];
      }
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        float vv[VEC];
        v_decode<CT>(vd[i], vv);
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[i] = ok[j] ? fmaf(pj[j], vv[j], acc[i]) : acc[i];
      }
    }
  };

  // prologue: NBUF - 1 tiles in flight
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(kb[u], vb[u], u);

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

  // merge the lanes that share a row (they hold different token columns)
  if constexpr (LPR >= 2) {
#pragma unroll
    for (int step = 1; step < LPR; step *= 2) {
      float mo, lo;
      float ao[NLOAD];
      if (step == 1) {
        mo = xor_lane<1>(m);
        lo = xor_lane<1>(l);
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) ao[i] = xor_lane<1>(acc[i]);
      } else {
        mo = xor_lane<2>(m);
        lo = xor_lane<2>(l);
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) ao[i] = xor_lane<2>(acc[i]);
      }
      const float mn = fmaxf(m, mo);
      const float fa = (m == mn) ? 1.0f : exp2_hw(m - mn);
      const float fb = (mo == mn) ? 1.0f : exp2_hw(mo - mn);
      l = l * fa + lo * fb;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) acc[i] = acc[i] * fa + ao[i] * fb;
      m = mn;
    }
  }

  bool bad = tw.bad;
  if constexpr (WAVES > 1) {
    // merge the wavefronts' states (lane i holds the same rows in every one)
    if (wave > 0) {
      float* st = s_state + ((wave - 1) * kWave + lane) * NSTATE;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) st[i] = acc[i];
      st[NLOAD] = m;
      st[NLOAD + 1] = bad ? -l - 1.0f : l;   // sign marks a bad table entry
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float* st = s_state + ((w - 1) * kWave + lane) * NSTATE;
      const float mo = st[NLOAD];
      float lo = st[NLOAD + 1];
      if (lo < 0.0f) {
        bad = true;
        lo = -lo - 1.0f;
      }
      const float mn = fmaxf(m, mo);
      const float fa = (m == mn) ? 1.0f : exp2_hw(m - mn);
      const float fb = (mo == mn) ? 1.0f : exp2_hw(mo - mn);
      l = l * fa + lo * fb;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) acc[i] = acc[i] * fa + st[i] * fb;
      m = mn;
    }
  }

  float res[NLOAD];
  if (bad) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) res[i] = __builtin_nanf("");
  } else if (ntiles_all <= 0) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) res[i] = 0.0f;
  } else {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) res[i] = (acc[i] / l) * p.v_scale;
  }
  write_row(res, lane % LPR == 0);
  if constexpr (PART) {
    if (lane == 0) {
      const int64_t idx = (int64_t)row * p.num_partitions + part;
      p.max_logits[idx] = bad ? __builtin_nanf("") : m * kLn2;
      p.exp_sums[idx] = bad ? __builtin_nanf("") : l;
    }
  }
}

template <typename QT, typename CT, int D, int BS, bool PART, int WAVES>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid = PART ? dim3(p.num_heads, p.num_seqs, p.num_partitions)
                        : dim3(p.num_heads * p.num_seqs, 1, 1);
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
