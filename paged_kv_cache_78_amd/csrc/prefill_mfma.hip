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
// heads per kv head, row r = token r / G, head r % G) are cut into workgroup
// units of ROWS = 4 wavefronts x R blocks of 16 rows.  A workgroup walks the
// keys in stages of 32 (two 16-key sub-tiles): its 256 threads copy the
// stage's K and V tiles (gathered through the block table) into LDS once, and
// every wavefront multiplies them with its R row blocks:
//
//   S^T [16 keys x 16 rows] = K [16 x D] . Q^T [D x 16]        (v_mfma 16x16x32)
//   O^T [16 dims x 16 rows] += V^T [16 x 32 keys] . P^T [32 x 16]  (v_mfma 16x16x32)
//
// so each K/V byte read from memory feeds 16 * 4 * R query rows, and each
// operand read from LDS feeds R products.  Lane (n, g) holds column n (one
// query row) and rows 4g..4g+3 of every S^T and O^T product, so a row's
// softmax state lives in the lanes of its column.  In the PV product the
// 8 contraction elements of lane group g are the keys 4g..4g+3 of both
// sub-tiles, which is where S^T put them: the weights go into the B operand
// without any exchange, and the V operand reads the matching token quads.
// The 16-byte granules of each K row in LDS are XOR-permuted by the key and
// V's token-quad regions are padded by 128 bytes, so that the operand reads
// hit every bank once.  The copies go from global memory straight into LDS
// (buffer loads with the lds bit), three stages in a ring.  Three workgroups share a CU
// (three wavefronts per SIMD: at most 168 registers each, and 3 x 52.75 KB of
// LDS at head size 128): a wavefront alone keeps its SIMD busy little more
// than half the time (the K/V reads from LDS, the product chains and the
// barrier each stall it), and the other two fill much of the rest.
//
// Work mapping: each XCD has a queue of work units (the chunks of its
// (sequence, kv head) items, one after the other, the chunk with more keys
// first, items by decreasing context), so the chunks of an item share that
// XCD's L2.  The workgroups are persistent, as many as are resident at once:
// workgroup b runs on XCD b % 8 (they go to the XCDs round robin) and walks
// that XCD's queue in rounds, without a new dispatch per unit.  The sum of a
// row's weights comes from the matrix core (an all-ones A operand).
//
// Weight precision, fp8 decoding and masking follow the decode kernels: P in
// f16 (f16 and fp8 caches) or split into two bf16 parts (bf16 caches); keys
// past a row's limit get a -inf logit and weight 0, V elements of tokens past
// the context are zeroed before the product (a NaN in an unused slot must not
// reach it), and table entries past the context are never used (a few past
// it, inside the row, may be read).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "mfma_common.h"
#include "pa_decode_common.h"
#include "pa_kernels.h"

// LDS stage buffers of the prefill ring (3 or 4)
#ifndef PA_PF_STAGES
#define PA_PF_STAGES 3
#endif

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfKeys = 32;           // keys per stage
constexpr int kXcds = 8;              // workgroups go to the XCDs round robin
constexpr int kMaxDevices = 64;
constexpr float kNegInfP = kMfmaNegInf;
constexpr float kSlackP = 8.0f;
// s_waitcnt immediates (gfx9-family encoding): vmcnt(0) with expcnt and
// lgkmcnt at their maxima (or in a vmcnt(n)), and lgkmcnt(0) alone
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// The block table through the constant address space: entries come in
// through scalar loads, whose waits do not hold back the vector loads.
typedef const __attribute__((address_space(4))) int32_t ConstTable;
typedef __attribute__((address_space(3))) u32x2_t LdsU32x2;

template <typename QT, typename CT, int D, int BS, int R>
struct PfShape {
  static constexpr int ESZ = CT::kBytes;
  static constexpr int NQK = D / 32;                 // QK products per sub-tile
  static constexpr int NPV = D / 16;                 // PV products per stage
  static constexpr int ROWB = D * ESZ;               // bytes of one key's K row
  static constexpr int GPR = ROWB / 16;              // 16-byte granules per K row
  static constexpr int KB = kPfKeys * ROWB;          // K bytes of a stage (= V bytes)
  static constexpr int NREG = KB / 1024;             // 1 KiB copy regions of K (and of V)
  static constexpr int KPR = 1024 / ROWB;            // keys per K region
  static constexpr int QB = 4 * ROWB;                // bytes of one token quad of V
  static constexpr int QPR = 1024 / QB;              // token quads per V region
  // one quad per region: pad regions by 128 bytes so that the quads read by
  // lane groups 0 and 1 fall in different banks
  static constexpr int VREG = 1024 + (QPR == 1 ? 128 : 0);
  static constexpr int STAGE = KB + NREG * VREG;
  static constexpr int NREGW = 2 * NREG / kPfWaves;  // copy regions per wavefront per stage
  static constexpr int ROWS = kPfWaves * 16 * R;     // query rows per workgroup
  static constexpr int TILE_BYTES = BS * D * ESZ;
  static_assert(NREGW >= 1 && 2 * NREG % kPfWaves == 0 && NREGW <= 15, "stage split");
  static_assert(kPfKeys % BS == 0, "a stage holds whole blocks");
};

// maximum of 8 values (NaN-propagating v_maximum3_f32, which needs no
// canonicalised operands)
__device__ __forceinline__ float max8(const float (&v)[8]) {
  const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]), v[2]);
  const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[3], v[4]), v[5]);
  const float c = __builtin_elementwise_maximum(v[6], v[7]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

template <typename QT, typename CT, int D, int BS, bool CAUSAL, int R>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_mfma_kernel(const PrefillParams p,
                                                                   int chunks, int units_x) {
  using Sh = PfShape<QT, CT, D, BS, R>;
  constexpr int ESZ = Sh::ESZ, NQK = Sh::NQK, NPV = Sh::NPV;
  constexpr int ROWB = Sh::ROWB, GPR = Sh::GPR, KB = Sh::KB, KPR = Sh::KPR;
  constexpr int QB = Sh::QB, QPR = Sh::QPR, VREG = Sh::VREG, STAGE = Sh::STAGE;
  constexpr int NREGW = Sh::NREGW, ROWS = Sh::ROWS, TILE_BYTES = Sh::TILE_BYTES;
  constexpr int BPS = kPfKeys / BS;   // blocks per stage
  constexpr int NST = PA_PF_STAGES;   // LDS ring: NST - 1 stages in flight while one computes
  static_assert(NST == 3 || NST == 4, "stage ring");
  using M = Mma<QT>;
  using MV = std::conditional_t<ESZ == 1, Mma<F16>, Mma<QT>>;
  constexpr bool kSplitP = ESZ == 2 && __is_same(QT, BF16);

  __shared__ __attribute__((aligned(16))) char s_kv[NST][STAGE];
  __shared__ __attribute__((aligned(16))) int32_t s_ent[2][64];   // table windows
  __shared__ int32_t s_bad[kPfWaves];   // a wavefront met a bad table entry

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;          // query row of the wavefront's row blocks
  const int g = lane >> 4;          // lane group
  const int H = p.num_heads;
  const int KVH = p.num_kv_heads;
  const int G = H / KVH;
  const int MB = p.max_blocks_per_seq;

  // Work units: the chunks of an item (sequence, kv head) all belong to the
  // XCD item % 8 and come one after the other in its queue, the chunk with
  // the most keys first (they share the item's K/V in that XCD's L2).  Up to
  // 64 sequences, each XCD's queue takes the sequences' items in the order of
  // decreasing context (longest work first, so that the queue ends with
  // short work); beyond that, in item order.  Each XCD's queue holds units_x
  // units (some past the items are empty).
  //
  // The workgroups are persistent: workgroup b runs on XCD b % 8 (workgroups
  // go to the XCDs round robin) and the SPX = gridDim.x / 8 workgroups of an
  // XCD walk its queue in rounds of SPX units: round r gives the i-th of
  // them unit r SPX + i, or r SPX + SPX - 1 - i in odd rounds, so that over
  // two rounds each takes one of the longer and one of the shorter units.
  // A unit starts as soon as the last one ends, with no new dispatch, and
  // the ranking of the sequences is done once.
  const int x = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int SPX = gridDim.x / kXcds;
  const bool ranked = p.num_seqs <= 64;
  // lane l: sequence l, its items on this XCD and the queue position of its
  // first unit (contexts ranked, ties: the lower index first)
  int rk_mult = 0, rk_pos = 0;
  if (ranked) {
    const int sl = lane < p.num_seqs ? lane : 0;
    const int kl = p.context_lens[sl];
    const int rr = ((x - sl * KVH) % kXcds + kXcds) % kXcds;   // its first kv head here
    rk_mult = lane < p.num_seqs && rr < KVH ? (KVH - 1 - rr) / kXcds + 1 : 0;
    const int64_t key = ((int64_t)kl << 6) | (63 - lane);
    for (int l2 = 0; l2 < p.num_seqs; ++l2) {
      const int klo = __builtin_amdgcn_readlane(kl, l2);
      const int m2 = __builtin_amdgcn_readlane(rk_mult, l2);
      const int64_t k2 = ((int64_t)klo << 6) | (63 - l2);
      rk_pos += k2 > key ? m2 * chunks : 0;
    }
  }

  // Unit j of this XCD's queue: its sequence s, chunk c (the chunk with the
  // most keys first) and kv head; false past the items.
  auto unit_at = [&](int j, int& s, int& c, int& kvh) -> bool {
    if (ranked) {
      const uint64_t hit =
          __builtin_amdgcn_ballot_w64(rk_mult > 0 && rk_pos <= j && j < rk_pos + rk_mult * chunks);
      const bool live = hit != 0;
      const int gl = live ? (int)__builtin_ctzll(hit) : 0;
      const int local = j - __builtin_amdgcn_readlane(rk_pos, gl);
      s = gl;
      c = chunks - 1 - local % chunks;
      kvh = ((x - s * KVH) % kXcds + kXcds) % kXcds + kXcds * (local / chunks);
      return live;
    }
    const int item = (j / chunks) * kXcds + x;
    const bool live = item < p.num_seqs * KVH;
    c = chunks - 1 - j % chunks;
    s = live ? item / KVH : 0;
    kvh = item % KVH;
    return live;
  };

  // Q^T operands: row block r's column n, dims 32 cc + 8 g .. +7 of chunk cc.
  // qready: they were loaded at the end of the last unit for this one.  With
  // bf16 queries or fp8 caches the next unit's Q is loaded at the end of each
  // unit, so its latency passes during the epilogue and the unit start
  // (interleaved timing: bf16 -2.0 to -2.5%, fp8 caches -2.5 to -3.8%); with
  // f16 queries over f16 caches the same was 0.8-1.5% slower, and Q is loaded
  // at the unit start.
  constexpr bool kQNext = !(__is_same(QT, F16) && ESZ == 2);
  u32x4_t qb[R][NQK];
  bool qready = false;
  for (int round = 0;; ++round) {
    const int jq = round * SPX + ((round & 1) ? SPX - 1 - slot : slot);
    if (jq >= units_x) break;
    // the last unit's LDS (stage buffers, table windows, the bad-entry flags)
    // is free once every wavefront is here: its LDS accesses are complete
    // (its copies were all waited for in its last stages), and the bare
    // barrier leaves the next unit's Q loads in flight
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const bool qpre = qready;
    qready = false;
    int s, c, kvh;
    const bool live = unit_at(jq, s, c, kvh);

    // The sequence's lengths and the table entries of its first three stages
    // are loaded at once (indices clamped into the row; entries past the
    // context are never used), and waited for together before any branch.
    constexpr int NPRE = NST;
    const int wblk = (16 * (wave & 1)) / BS;   // the stage block whose half this wavefront copies
    int epre[NPRE];
    const int32_t q0 = p.cu_seqlens_q[s];
    const int32_t q1 = p.cu_seqlens_q[s + 1];
    const int K = p.context_lens[s];
    {
      ConstTable* trow = (ConstTable*)(p.block_table + (int64_t)s * MB);
#pragma unroll
      for (int i = 0; i < NPRE; ++i) epre[i] = trow[min(i * BPS + wblk, MB - 1)];
    }
    const int total_q = p.total_q, max_seqlen_q = p.max_seqlen_q;
    const int64_t q_token_stride = p.q_token_stride, num_blocks = p.num_blocks;
    asm volatile("" ::"s"(q0), "s"(q1), "s"(K), "s"(total_q), "s"(max_seqlen_q));
    asm volatile("" ::"s"(q_token_stride), "s"(num_blocks));
#pragma unroll
    for (int i = 0; i < NPRE; ++i) asm volatile("" ::"s"(epre[i]));
    if (!live) continue;
    const int nq = q1 - q0;
    // packed rows outside [0, total_q) are never touched
    if (q0 < 0 || q1 > total_q || nq <= 0) continue;
    const int rows = nq * G;
    const int row0 = c * ROWS;
    if (row0 >= rows) continue;
    const bool bad_len = K < 0 || K > MB * BS || nq > max_seqlen_q;

    // this lane's rows (one per row block) and the keys each attends: 0 .. lim-1
    int qi[R], hh[R], lim[R];
    bool ok_row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + wave * 16 * R + 16 * r + n;
      ok_row[r] = row < rows;
      qi[r] = ok_row[r] ? row / G : 0;
      hh[r] = kvh * G + (ok_row[r] ? row % G : 0);
      int lm = 0;
      if (ok_row[r] && !bad_len) lm = CAUSAL ? min(K, K - nq + qi[r] + 1) : K;
      lim[r] = max(lm, 0);
    }
    // the workgroup's stages: up to its last row's limit (limits grow with the row)
    int wg_lim = 0;
    if (!bad_len) {
      const int last_q = (min(row0 + ROWS, rows) - 1) / G;
      wg_lim = max(CAUSAL ? min(K, K - nq + last_q + 1) : K, 0);
    }
    const int nstages = (wg_lim + kPfKeys - 1) / kPfKeys;
    const int ctx_blocks = (K + BS - 1) / BS;           // table entries that may be read

    auto store_rows = [&](const float4_t (&o)[R][NPV]) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!ok_row[r]) continue;
        uint16_t* dst =
            reinterpret_cast<uint16_t*>(p.out) + ((int64_t)(q0 + qi[r]) * H + hh[r]) * D;
        // lane (n, g) holds dims 16 jj + 4g .. +3 of product jj
#pragma unroll
        for (int jj = 0; jj < NPV; ++jj) {
          const uint32_t w0 = (uint32_t)to_bits16<QT>(o[r][jj][0]) |
                              ((uint32_t)to_bits16<QT>(o[r][jj][1]) << 16);
          const uint32_t w1 = (uint32_t)to_bits16<QT>(o[r][jj][2]) |
                              ((uint32_t)to_bits16<QT>(o[r][jj][3]) << 16);
          *reinterpret_cast<u32x2_t*>(dst + 16 * jj + 4 * g) = u32x2_t{w0, w1};
        }
      }
    };

    if (bad_len) {
      float4_t o[R][NPV];
      const float nanv = __builtin_nanf("");
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int jj = 0; jj < NPV; ++jj) o[r][jj] = float4_t{nanv, nanv, nanv, nanv};
      store_rows(o);
      continue;
    }


    // ---- staging: the stage's K and V tiles, copied global -> LDS ----
    // A copy instruction puts lane i's 16 bytes at LDS base + 16 i: each
    // wavefront fills NREGW regions of 1 KiB per stage, wavefronts 0-1 those of
    // K and 2-3 those of V.  K region r holds keys r*KPR .. with the 16-byte
    // granules of key kk XOR-permuted by kk % GPR (so the 16 keys a K operand
    // read touches land in different banks); V region r holds token quads
    // r*QPR .. in the tile layout.
    const int32_t* table_v = p.block_table + (int64_t)s * MB;
    const bool copies_k = wave < 2;
    const char* cache = reinterpret_cast<const char*>(copies_k ? p.k_cache : p.v_cache) +
                        (int64_t)kvh * TILE_BYTES;
    const int64_t block_stride = (int64_t)KVH * TILE_BYTES;
    const uint32_t nb32 = (uint32_t)min(num_blocks, (int64_t)INT32_MAX);
    bool bad_entry = false;

    // The regions of a wavefront are half a stage: the 16 keys 16 (wave % 2)
    // .. of K, or the 4 token quads (16 tokens) of V starting there, always
    // inside one cache block (block wblk of the stage, at byte offset roff0),
    // consecutive 1 KiB apart in the source.  So a stage's copy needs one
    // table entry per wavefront, and the sources are block address + per-lane
    // offsets fixed for the loop.  The block address goes into a buffer
    // descriptor (scalar registers) and each region's offset is one 32-bit
    // register: 64-bit lane addresses would take twice the registers, and
    // with them the kernel spilled at three wavefronts per SIMD.
    const int half = wave & 1;
    const int roff0 = copies_k ? ((16 * half) % BS) * ROWB : ((4 * half) % (BS / 4)) * QB;
    const int rdst0 = copies_k ? wave * NREGW * 1024 : KB + half * NREGW * VREG;
    const int rstep = copies_k ? 1024 : VREG;
    const int b16 = 16 * lane;
    uint32_t loff[NREGW];                               // region i: source byte offset
#pragma unroll
    for (int i = 0; i < NREGW; ++i) {
      if (copies_k) {
        const int kk = (wave * NREGW + i) * KPR + b16 / ROWB;   // key within the stage
        loff[i] = i * 1024 + (b16 / ROWB) * ROWB + (((b16 % ROWB) / 16) ^ (kk % GPR)) * 16;
      } else {
        loff[i] = i * 1024 + b16;
      }
    }

    // copies this wavefront's half of stage t into the buffer at byte offset
    // boff; e: the table entry of its block.  A block past the context or with
    // a bad entry reads block 0 (any valid address: its keys are masked and
    // its V elements zeroed).
    auto stage_copy = [&](int t, int boff, int e) {
      uint32_t ph = (uint32_t)e;
      if (t * BPS + wblk >= ctx_blocks) {
        ph = 0;
      } else if (ph >= nb32) {                          // negative or past the pool
        bad_entry = true;
        ph = 0;
      }
      const char* base = cache + (int64_t)ph * block_stride + roff0;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, NREGW * 1024);
#pragma unroll
      for (int i = 0; i < NREGW; ++i) {
        // named locals: an array element passed straight to the builtin made
        // the host pass drop the kernels' launch stubs
        char* dst = &s_kv[0][0] + boff + rdst0 + i * rstep;
        const uint32_t lo = loff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst,
                                                 16, lo, 0, 0, 0);
      }
    };

    // Table entries inside the loop come from LDS: windows of 64 entries are
    // copied in by wavefront 0 into a ring of two, 2 NST - 2 stages before their
    // first use (the wait NST - 2 stages later covers the copy, and that
    // stage's barrier publishes it).  Lane l copies the entry of block 64 w + l,
    // clamped into the context (entries past it are never used).  A scalar
    // load in flight would make every LDS wait of a stage wait for it too.
    constexpr int SPW = 64 / BPS;                       // stages per window
    auto window_copy = [&](int w) {
      const int lb = max(min(64 * w + lane, ctx_blocks - 1), 0);
      const int32_t* src = table_v + lb;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)s_ent[w & 1],
                                       4, 0, 0);
    };
    // the entry of this wavefront's block of stage t, read from its window
    auto entries_read = [&](int t) -> int { return s_ent[(t / SPW) & 1][(t % SPW) * BPS + wblk]; };
    // entry of stage t < NST, from those loaded up front
    auto entries_pre = [&](int t) -> int { return epre[t]; };

    // ---- the products ----
    // Row limits are non-decreasing in the row, so the wavefront's valid rows
    // attend at least keys 0 .. wmin-1 and at most 0 .. wmax-1: stages below
    // wmin need no logit mask, stages from wmax on give every row weight 0.
    const int wrow0 = row0 + wave * 16 * R;
    const int wrow1 = min(wrow0 + 16 * R, rows) - 1;
    auto lim_of = [&](int row) {
      return CAUSAL ? max(min(K, K - nq + row / G + 1), 0) : K;
    };
    const int wmin = wrow0 <= wrow1 ? lim_of(wrow0) : 0;
    const int wmax = wrow0 <= wrow1 ? lim_of(wrow1) : 0;

    // Logits are taken as raw products times |scale|: a negative scale flips
    // the sign of Q (exact), so the row maximum of the raw products scales to
    // the maximum of the logits.
    // A zero scale takes the smallest normal instead: every logit is then
    // below 2^-100 in magnitude, its weight exactly 1, and a masked product
    // (-inf) still gives -inf.
    const float sl = fmaxf(fabsf(p.qk_scale_log2), __FLT_MIN__);

    // running maximum starts finite, so that exp2(logit - m) needs no guard:
    // a masked logit (-inf) gives 0 whatever m is.  The sum of the weights,
    // as they enter the PV product, comes with 16-bit caches from the matrix
    // core: one more product per row block, of an all-ones A operand with the
    // packed weights, leaves in every lane of column n the sum of row n's
    // weights (lacc).  With fp8 caches, whose operand decoding needs more
    // registers, each lane sums its own 8 weights per stage with v_dot2
    // (exact products with 1, an fp32 sum: lsum), and the 4 lanes of a row add
    // theirs at the end; lacc and its all-ones operand (12 registers) would
    // otherwise spill at three wavefronts per SIMD.
    constexpr bool kSumValu = ESZ == 1;
    float m[R];
    float4_t lacc[R];
    float lsum[R];
    float4_t acc[R][NPV];
    const u32x4_t ones = u32x4_t{MV::kOne2, MV::kOne2, MV::kOne2, MV::kOne2};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = -__FLT_MAX__;
      lacc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
      lsum[r] = 0.0f;
#pragma unroll
      for (int jj = 0; jj < NPV; ++jj) acc[r][jj] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // K operand of sub-tile u, chunk cc: key 16u + n, dims 32 cc + 8 g .. +7
    auto k_operand = [&](const char* kb, int u, int cc) -> u32x4_t {
      const int kk = 16 * u + n;
      const int byte = (32 * cc + 8 * g) * ESZ;
      const char* src = kb + kk * ROWB + (((byte / 16) ^ (kk % GPR)) * 16) + byte % 16;
      if constexpr (ESZ == 2) {
        return *reinterpret_cast<const u32x4_t*>(src);
      } else {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(src);
        return u32x4_t{M::template fp8x2<false>(w[0]), M::template fp8x2<true>(w[0]),
                       M::template fp8x2<false>(w[1]), M::template fp8x2<true>(w[1])};
      }
    };
    // V operand of product jj: dim 16 jj + n, keys 4g..4g+3 (quad g) and
    // 16+4g..16+4g+3 (quad 4+g) of the stage
    auto quad_at = [&](const char* vb, int q) {
      return vb + (q / QPR) * VREG + (q % QPR) * QB;
    };
    auto v_operand = [&](const char* vb, int jj) -> u32x4_t {
      const char* a = quad_at(vb, g) + (16 * jj + n) * 4 * ESZ;
      const char* b2 = quad_at(vb, 4 + g) + (16 * jj + n) * 4 * ESZ;
      if constexpr (ESZ == 2) {
        // volatile: keeps each half a read of its own, straight into its
        // registers (paired reads of neighbouring products need moves)
        const u32x2_t x = *(const volatile LdsU32x2*)a;
        const u32x2_t y = *(const volatile LdsU32x2*)b2;
        return u32x4_t{x[0], x[1], y[0], y[1]};
      } else {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(a);
        const uint32_t y = *reinterpret_cast<const uint32_t*>(b2);
        return u32x4_t{MV::template fp8x2<false>(x), MV::template fp8x2<true>(x),
                       MV::template fp8x2<false>(y), MV::template fp8x2<true>(y)};
      }
    };

    // One stage.  The weights come from one of two paths (masked: some row of
    // the wavefront stops inside the stage, its logits past the row limit are
    // -inf; unmasked: every key counts for every valid row and the logits go
    // straight from the products to exp2), then the accumulators meet a single
    // product path, so each product updates them in place.  The weights of
    // both row blocks are taken first, then the V operands are read from LDS
    // one ahead of their products (operand jj + 1 is in flight while jj's two
    // products run): a wavefront holds two V operands instead of all NPV,
    // which fits the kernel in the registers of three wavefronts per SIMD (the
    // latency a wavefront leaves exposed is covered by the other two).
    auto compute = [&](bool masked, int t, int boff) {
      const char* kb = &s_kv[0][0] + boff;
      const char* vb = kb + KB;
      const int key0 = t * kPfKeys;
      // raw products of keys key0 + 16u + 4g + i, per row block
      float4_t sc[R][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][u] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NQK; ++cc) {
          const u32x4_t ka = k_operand(kb, u, cc);
#pragma unroll
          for (int r = 0; r < R; ++r) sc[r][u] = M::qk(ka, qb[r][cc], sc[r][u]);
        }
      }
      // Masked stage (some row of the wavefront stops inside it): products of
      // keys past a row's limit become -inf, so their logits (times sl > 0)
      // are -inf and their weights 0.  Then the row maxima of the stage.
      if (masked) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = key0 + 16 * (i >> 2) + 4 * g + (i & 3);
            sc[r][i >> 2][i & 3] = key < lim[r] ? sc[r][i >> 2][i & 3] : kNegInfP;
          }
      }
      float mt[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sc[r][i >> 2][i & 3];
        mt[r] = max8(x) * sl;
      }
      bool grow = false;
#pragma unroll
      for (int r = 0; r < R; ++r) grow |= mt[r] > m[r] + kSlackP;
      // Lazy rescale: the running maximum moves only when some row's stage
      // maximum passes it by more than the slack (weights stay below 2^slack);
      // then the accumulators are rescaled.  Decided before any weight is
      // taken, so that the weights, their packing and the products that use
      // them form one block.
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float mm = mt[r];
          mm = __builtin_elementwise_maximum(mm, __shfl_xor(mm, 16, 64));
          mm = __builtin_elementwise_maximum(mm, __shfl_xor(mm, 32, 64));
          const float mn = fmaxf(m[r], mm);
          const float alpha = exp2_hw(m[r] - mn);
          m[r] = mn;
          lacc[r] *= alpha;
          lsum[r] *= alpha;
#pragma unroll
          for (int jj = 0; jj < NPV; ++jj) acc[r][jj] *= alpha;
        }
      }
      // per row block: the weights exp2(logit - m), packed as the PV B
      // operand (bf16 caches: and the remainder of each weight, packed again),
      // and the weights' sum
      u32x4_t pb[R], pl[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pr[i] = exp2_hw(__builtin_fmaf(sc[r][i >> 2][i & 3], sl, -m[r]));
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = MV::pack_pk(pr[2 * k], pr[2 * k + 1]);
        pb[r] = u32x4_t{w[0], w[1], w[2], w[3]};
        pl[r] = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (kSplitP) {
          uint32_t v2[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            v2[k] = MV::pack_pk(pr[2 * k] - MV::lo(w[k]), pr[2 * k + 1] - MV::hi(w[k]));
          pl[r] = u32x4_t{v2[0], v2[1], v2[2], v2[3]};
        }
        if constexpr (kSumValu) {
#pragma unroll
          for (int k = 0; k < 4; ++k) lsum[r] = MV::sum2(w[k], lsum[r]);
        } else {
          lacc[r] = MV::qk(ones, pb[r], lacc[r]);
          if constexpr (kSplitP) lacc[r] = MV::qk(ones, pl[r], lacc[r]);
        }
      }
      // the PV products, V operand by V operand
      u32x4_t va = v_operand(vb, 0);
#pragma unroll
      for (int jj = 0; jj < NPV; ++jj) {
        u32x4_t vn = va;
        if (jj + 1 < NPV) vn = v_operand(vb, jj + 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r][jj] = MV::qk(va, pb[r], acc[r][jj]);
          if constexpr (kSplitP) acc[r][jj] = MV::qk(va, pl[r], acc[r][jj]);
        }
        va = vn;
      }
    };

    // V elements of tokens past the context, in the last stage when the
    // context ends inside it: zeroed in LDS by the wavefronts that copied V,
    // once their copies have landed and before the barrier (a NaN there must
    // not reach the product, even with weight 0).  Lane pairs (dim, quad) of
    // the wavefront's regions.
    auto zero_v_tail = [&](int t, int boff) {
      const int j0 = K - t * kPfKeys;                   // first local token past the context
      constexpr int QW = NREGW * QPR;                   // token quads of the wavefront
      const int vr0 = (wave - 2) * NREGW;               // its first V region
      for (int idx = lane; idx < QW * D; idx += 64) {
        const int ql = idx / D, d = idx % D;
        const int vr = vr0 + ql / QPR;
        const int q = vr * QPR + ql % QPR;              // quad within the stage
        if (4 * q + 3 < j0) continue;
        char* at = &s_kv[0][0] + boff + KB + vr * VREG + (ql % QPR) * QB + d * 4 * ESZ;
        if constexpr (ESZ == 2) {
          u32x2_t v = *reinterpret_cast<u32x2_t*>(at);
          const int e0 = j0 - 4 * q;                    // first element to clear (may be <= 0)
          v[0] &= (e0 > 0 ? 0x0000FFFFu : 0u) | (e0 > 1 ? 0xFFFF0000u : 0u);
          v[1] &= (e0 > 2 ? 0x0000FFFFu : 0u) | (e0 > 3 ? 0xFFFF0000u : 0u);
          *reinterpret_cast<u32x2_t*>(at) = v;
        } else {
          uint32_t v = *reinterpret_cast<uint32_t*>(at);
          const int e0 = j0 - 4 * q;
          v &= (e0 > 0 ? 0x000000FFu : 0u) | (e0 > 1 ? 0x0000FF00u : 0u) |
               (e0 > 2 ? 0x00FF0000u : 0u) | (e0 > 3 ? 0xFF000000u : 0u);
          *reinterpret_cast<uint32_t*>(at) = v;
        }
      }
    };

    // Stage 0's copies, then Q, waited for together before the next stages' copies
    // and the loop (a load the compiler still counts as pending at the loop
    // entry would make every stage wait for all of its copies in flight; it
    // does not count the copies when it checks an explicit wait against Q).
    int ecur = entries_pre(NST - 1);                    // entry of stage t + NST - 1
    if (nstages > 0) {
      stage_copy(0, 0, entries_pre(0));
      if (wave == 0 && nstages > 3) window_copy(0);
    }
    if (!qpre) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)(q0 + qi[r]) * q_token_stride + (int64_t)hh[r] * D) * 2;
#pragma unroll
        for (int cc = 0; cc < NQK; ++cc)
          qb[r][cc] = ok_row[r] ? *reinterpret_cast<const u32x4_t*>(qrow + (32 * cc + 8 * g) * 2)
                                : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (p.qk_scale_log2 < 0.0f) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int cc = 0; cc < NQK; ++cc) qb[r][cc] ^= 0x80008000u;
    }
#pragma unroll
    for (int i = 1; i < NST - 1; ++i)
      if (nstages > i) stage_copy(i, i * STAGE, entries_pre(i));

    // Stage t is copied NST - 1 stages ahead.  Waits are explicit (the
    // barrier here is the bare instruction, whose implied fence would wait for
    // every copy in flight): each lane waits for its own copies of stage t
    // (those of the next NST - 2 stages may stay in flight) and for its LDS
    // reads of stage t-1, then the barrier makes stage t complete for all and
    // frees stage t-1's buffer, which receives stage t + NST - 1.  Every
    // wavefront copies and meets every barrier; it computes only the stages
    // some row of it attends.  The buffers rotate: stage t in buffer t % NST.
    // (Four buffers measured no faster than three: the copies arrive in time,
    // and the waits at the barrier are the wavefronts waiting for each other.)
    int cb = 0, nb = (NST - 1) * STAGE;                 // byte offsets: compute, copy
    int ev = 0;
    auto stage_begin = [&](int t) {
      if (t + NST - 2 < nstages) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0 | ((NST - 2) * NREGW));
      } else if (NST == 4 && t + 1 < nstages) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0 | NREGW);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (!copies_k && t * kPfKeys + kPfKeys > K) zero_v_tail(t, cb);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (t > 0) {                                      // entries read in the last stage
        ecur = __builtin_amdgcn_readfirstlane(ev);
      }
      if (t + NST - 1 < nstages) {
        // the window of stage t + 2 NST - 2 when it opens one: its copy
        // precedes this stage's copies, so the wait NST - 2 stages on covers
        // it, and the entries of its first stage are read at the end of that
        // stage
        constexpr int WA = 2 * NST - 2;
        if (wave == 0 && t + WA < nstages && (t + WA) % SPW == 0) window_copy((t + WA) / SPW);
        stage_copy(t + NST - 1, nb, ecur);
      }
    };
    auto stage_end = [&](int t) {
      // entries of stage t + NST, for the next stage's copy (its window
      // arrived with this stage's barrier)
      if (t + NST < nstages) ev = entries_read(t + NST);
      cb = cb == (NST - 1) * STAGE ? 0 : cb + STAGE;
      nb = nb == (NST - 1) * STAGE ? 0 : nb + STAGE;
    };
    // The stages this wavefront computes come first, then those it only
    // copies (two loops, so that no path of the first leaves the accumulators
    // as they were, which would cost a copy of them per stage).
    const int wstages = min(nstages, (wmax + kPfKeys - 1) / kPfKeys);
    int t = 0;
    for (; t < wstages; ++t) {
      stage_begin(t);
      compute(t * kPfKeys + kPfKeys > wmin, t, cb);
      stage_end(t);
    }
    for (; t < nstages; ++t) {
      stage_begin(t);
      stage_end(t);
    }

    // The next unit's Q, into the registers this unit no longer needs, when
    // that unit will compute (the same checks as at its start; nothing is
    // loaded for a unit that writes no rows or only NaN rows)
    if constexpr (kQNext) {
      const int round_n = round + 1;
      const int jn = round_n * SPX + ((round_n & 1) ? SPX - 1 - slot : slot);
      if (jn < units_x) {
        int sn, cn, kn;
        if (unit_at(jn, sn, cn, kn)) {
          const int32_t a0 = p.cu_seqlens_q[sn];
          const int32_t a1 = p.cu_seqlens_q[sn + 1];
          const int Kn = p.context_lens[sn];
          const int nqn = a1 - a0;
          const int rowsn = nqn * G;
          const int row0n = cn * ROWS;
          if (a0 >= 0 && a1 <= total_q && nqn > 0 && row0n < rowsn &&
              !(Kn < 0 || Kn > MB * BS || nqn > max_seqlen_q)) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const int row = row0n + wave * 16 * R + 16 * r + n;
              const bool okr = row < rowsn;
              const int qin = okr ? row / G : 0;
              const int hn = kn * G + (okr ? row % G : 0);
              const char* qrow = reinterpret_cast<const char*>(p.q) +
                                 ((int64_t)(a0 + qin) * q_token_stride + (int64_t)hn * D) * 2;
#pragma unroll
              for (int cc = 0; cc < NQK; ++cc)
                qb[r][cc] = okr ? *reinterpret_cast<const u32x4_t*>(qrow + (32 * cc + 8 * g) * 2)
                                : u32x4_t{0u, 0u, 0u, 0u};
            }
            qready = true;
          }
        }
      }
    }
    // A bad table entry met by any wavefront (each checks the blocks it
    // copies) makes the workgroup's rows NaN; a row with no key gives zeros.
    // The barrier waits for LDS only, leaving the next unit's Q in flight.
    s_bad[wave] = bad_entry ? 1 : 0;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const bool bad_any = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
    float4_t o[R][NPV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float lt = lacc[r][0];
      if constexpr (kSumValu) {
        lt = lsum[r];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
      }
      const float inv = bad_any ? __builtin_nanf("") : (lt > 0.0f ? p.v_scale / lt : 0.0f);
#pragma unroll
      for (int jj = 0; jj < NPV; ++jj) o[r][jj] = acc[r][jj] * inv;
    }
    store_rows(o);
  }
}

constexpr int kPfRowBlocks = 2;       // row blocks of 16 per wavefront

// Workgroups of kernel `kern` resident at once on the current device (its
// CUs times the workgroups one CU holds), looked up once per device.
template <typename Kern>
int resident_workgroups(Kern kern, std::atomic<int> (&cache)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPfThreads, 0) != hipSuccess)
    return 0;
  n = cus * per_cu;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename QT, typename CT, int D, int BS, bool CAUSAL>
hipError_t launch_grid(const PrefillParams& p, int chunks, int64_t units_x, hipStream_t stream) {
  static std::atomic<int> resident[kMaxDevices];
  auto kern = prefill_mfma_kernel<QT, CT, D, BS, CAUSAL, kPfRowBlocks>;
  const int n = resident_workgroups(kern, resident);
  if (n <= 0) return hipErrorInvalidDevice;
  // as many workgroups as are resident at once, a multiple of the XCD count
  // (at least one per XCD), never more than there are units
  const int64_t per_x = std::min<int64_t>(units_x, std::max(n / kXcds, 1));
  hipLaunchKernelGGL(kern, dim3((unsigned)(per_x * kXcds)), dim3(kPfThreads), 0, stream, p, chunks,
                     (int)units_x);
  return hipGetLastError();
}

template <typename QT, typename CT, int D, int BS>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  constexpr int ROWS = PfShape<QT, CT, D, BS, kPfRowBlocks>::ROWS;
  const int G = p.num_heads / p.num_kv_heads;
  const int64_t rows = (int64_t)p.max_seqlen_q * G;
  const int64_t chunks = (rows + ROWS - 1) / ROWS;
  const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t groups = (items + kXcds - 1) / kXcds;
  const int64_t units_x = groups * chunks;
  if (units_x * kXcds > INT32_MAX) return hipErrorInvalidConfiguration;
  return p.causal ? launch_grid<QT, CT, D, BS, true>(p, (int)chunks, units_x, stream)
                  : launch_grid<QT, CT, D, BS, false>(p, (int)chunks, units_x, stream);
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
