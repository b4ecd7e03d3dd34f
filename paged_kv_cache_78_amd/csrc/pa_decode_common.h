// Pieces shared by the decode kernels: the block-table window and the
// longest-first order of sequences.
#pragma once

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// Block-table window of one wavefront.  Entries [cbase, cbase + 64) of the
// range's table slice sit one per lane in `cur`, the next 64 in `nxt` (loaded
// a chunk ahead).  Loads go through a buffer descriptor sized to the slice, so
// lanes past the end read 0 without branches and nothing waits on the load
// until the chunk is used.  Entries outside [0, num_blocks) are replaced by 0
// before any address is formed and set `bad`.
struct TableWindow {
  __amdgpu_buffer_rsrc_t rsrc;
  int ntiles;
  int64_t num_blocks;
  int cbase;
  int cur;
  int nxt;
  bool bad;

  __device__ __forceinline__ int raw(int first, int lane) {
    return (int)buffer_load4(rsrc, (uint32_t)(first + lane) * 4u);
  }
  __device__ __forceinline__ int sanitize(int first, int lane, int v) {
    const bool inrange = (first + lane) < ntiles;
    const bool b = inrange && (v < 0 || (int64_t)v >= num_blocks);
    bad |= __builtin_amdgcn_ballot_w64(b) != 0;
    return b ? 0 : v;
  }
  __device__ __forceinline__ void init(const int32_t* slice, int n, int64_t nb, int lane) {
    rsrc = make_rsrc(slice, (uint32_t)(n > 0 ? n : 0) * 4u);
    ntiles = n;
    num_blocks = nb;
    cbase = 0;
    bad = false;
    cur = sanitize(0, lane, raw(0, lane));
    nxt = raw(64, lane);
  }
  __device__ __forceinline__ void init(const int32_t* slice, int n, int64_t nb, int lane, int*) {
    init(slice, n, nb, lane);
  }
  // Physical block of tile t (wave-uniform, t < ntiles, called with t
  // increasing by one).
  __device__ __forceinline__ int phys(int t, int lane) {
    if (t - cbase == 64) {
      cbase += 64;
      cur = sanitize(cbase, lane, nxt);
      nxt = raw(cbase + 64, lane);
    }
    return __builtin_amdgcn_readlane(cur, t - cbase);
  }
};

// The same window staged through LDS: each chunk of 64 entries is loaded as
// above (one per lane, the next chunk a chunk ahead), checked, written to the
// wavefront's 64-entry LDS slice, and every tile reads its entry back with one
// LDS load at a wave-uniform address.  Built with PA_TABLE_LDS=1 so that
// bench.py can compare it with the register window.
struct TableLds {
  TableWindow w;
  int* s;

  __device__ __forceinline__ void init(const int32_t* slice, int n, int64_t nb, int lane,
                                       int* lds) {
    w.init(slice, n, nb, lane);
    s = lds;
    s[lane] = w.cur;
    __builtin_amdgcn_wave_barrier();
  }
  __device__ __forceinline__ int phys(int t, int lane) {
    if (t - w.cbase == 64) {
      w.cbase += 64;
      w.cur = w.sanitize(w.cbase, lane, w.nxt);
      w.nxt = w.raw(w.cbase + 64, lane);
      __builtin_amdgcn_wave_barrier();
      s[lane] = w.cur;
      __builtin_amdgcn_wave_barrier();
    }
    return __builtin_amdgcn_readfirstlane(s[t - w.cbase]);
  }
};

#ifndef PA_TABLE_LDS
#define PA_TABLE_LDS 0
#endif
#if PA_TABLE_LDS
using TableSlice = TableLds;
__device__ __forceinline__ bool table_bad(const TableLds& t) { return t.w.bad; }
#else
using TableSlice = TableWindow;
__device__ __forceinline__ bool table_bad(const TableWindow& t) { return t.bad; }
#endif
// LDS the table slices of a workgroup of `waves` wavefronts take (ints)
constexpr int table_lds_ints(int waves) { return PA_TABLE_LDS ? waves * kWave : 1; }

// Longest-first order of sequences, computed by every workgroup of a
// one-pass launch from context_lens alone (no workspace, no host sync).
// Workgroups are dispatched in index order and spread over the compute units,
// so handing the longest contexts to the first workgroups evens out the work
// each compute unit receives.  Key: number of blocks (clamped to 255),
// descending; ties keep sequence order.  Counting sort over 256 keys in LDS,
// one wavefront.  Returns the sequence at position `rank`.
constexpr int kSchedKeys = 256;

__device__ __forceinline__ int sched_key(int len, int block_size) {
  const int nb = len > 0 ? (len + block_size - 1) / block_size : 0;
  return (kSchedKeys - 1) - (nb < kSchedKeys - 1 ? nb : kSchedKeys - 1);
}

// Up to kCachedSeqs sequences, each lane keeps the lengths it loaded (one
// load per sequence, all issued at once) for the second pass and for the
// returned length; beyond that, they are loaded again.
constexpr int kCachedSeqs = 4 * kWave;

__device__ __forceinline__ int seq_by_rank(const int32_t* context_lens, int num_seqs,
                                           int block_size, int rank, int* hist, int lane,
                                           int& len) {
  constexpr int NC = kCachedSeqs / kWave;
  const bool cached = num_seqs <= kCachedSeqs;
  int cl[NC];
  if (cached) {
    // indices clamped into the array, so every load is issued unconditionally
#pragma unroll
    for (int i = 0; i < NC; ++i) cl[i] = context_lens[min(lane + i * kWave, num_seqs - 1)];
  }
#pragma unroll
  for (int i = 0; i < kSchedKeys / kWave; ++i) hist[lane + i * kWave] = 0;
  __syncthreads();
  if (cached) {
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane + i * kWave < num_seqs) atomicAdd(&hist[sched_key(cl[i], block_size)], 1);
  } else {
    for (int s = lane; s < num_seqs; s += kWave)
      atomicAdd(&hist[sched_key(context_lens[s], block_size)], 1);
  }
  __syncthreads();
  // lane owns keys [4 lane, 4 lane + 4): exclusive prefix over lanes
  int c[4];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = hist[4 * lane + i];
    tot += c[i];
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  const int excl = incl - tot;
  const uint64_t own = __builtin_amdgcn_ballot_w64(excl <= rank && rank < incl);
  const int owner = own ? (int)__builtin_ctzll(own) : 0;
  // first of this lane's keys whose range holds `rank` (empty keys skipped)
  int key = 4 * lane + 3, start = excl;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!found) {
      if (rank < start + c[i]) {
        key = 4 * lane + i;
        found = true;
      } else {
        start += c[i];
      }
    }
  }
  key = __builtin_amdgcn_readlane(key, owner);
  int target = rank - __builtin_amdgcn_readlane(start, owner);
  // the target-th sequence (in index order) carrying that key
  if (cached) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bool match = lane + i * kWave < num_seqs && sched_key(cl[i], block_size) == key;
      const uint64_t m = __builtin_amdgcn_ballot_w64(match);
      const int cnt = __builtin_popcountll(m);
      if (target < cnt) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(match && below == target);
        const int l = (int)__builtin_ctzll(hit);
        len = __builtin_amdgcn_readlane(cl[i], l);
        return i * kWave + l;
      }
      target -= cnt;
    }
  } else {
    for (int base = 0; base < num_seqs; base += kWave) {
      const int s = base + lane;
      const bool match = s < num_seqs && sched_key(context_lens[s], block_size) == key;
      const uint64_t m = __builtin_amdgcn_ballot_w64(match);
      const int cnt = __builtin_popcountll(m);
      if (target < cnt) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(match && below == target);
        const int sq = base + (int)__builtin_ctzll(hit);
        len = context_lens[sq];
        return sq;
      }
      target -= cnt;
    }
  }
  len = context_lens[0];
  return 0;   // rank >= num_seqs: not reached for valid launches
}

// Position in the longest-first list that workgroup b of a one-pass launch of
// the matrix-core kernel takes (the vector-ALU kernel's is die_position
// below; the die weighting made the matrix-core kernels 1-4% slower, as their
// dies finish within 3-5% of each other).  Workgroups go to compute units
// round-robin, so consecutive strata of `units` workgroups
// alternate direction (a snake): each compute unit then gets one long and
// one short item from every pair of strata instead of always the longer one.
__device__ __forceinline__ int snake_position(int b, int total, int units) {
  const int k = b / units;
  const int i = b - k * units;
  if ((k & 1) == 0) return b;
  const int m = min(units, total - k * units);   // size of this stratum
  return k * units + (m - 1 - i);
}

// Position in the list of work items (one pass: the longest-first list;
// partitions: partition-major order) that workgroup b of a launch of the
// vector-ALU kernel takes.  Workgroups go to the dies (XCDs) round robin:
// workgroup b runs on die b % kDies as the j-th workgroup there, j = b / kDies.
// The odd-numbered dies of this part stream more slowly than the even ones
// (with equal work they finish 5-10% later; a streaming read with 6% more
// tiles on the even dies and 6% fewer on the odd ones ran 3-4% faster), so
// positions are handed out in the order of a virtual time that advances by
// die_cost(x) per workgroup of die x: workgroup (x, j) sits at
// (2j + 1) die_cost(x), and its position is the number of workgroups of all
// dies at an earlier time (equal times: the lower die first).  Every die still
// takes its items in list order, and an even die takes die_cost(1) /
// die_cost(0) times as many items as an odd one.  The launch has
// kDies * die_workgroups(items) workgroups; those whose position is `items` or
// more are spares and exit at once.
constexpr int kDies = 8;
__host__ __device__ constexpr int die_cost(int x) { return (x & 1) ? 53 : 47; }
// workgroups per die: an even die's share of the items, rounded up
__host__ __device__ constexpr int die_workgroups(int items) {
  return (int)(((int64_t)items * die_cost(1) * 2 / (die_cost(0) + die_cost(1)) + kDies - 1) /
               kDies);
}
__device__ __forceinline__ int die_position(int b, int n) {
  const int x = b % kDies;
  const int j = b / kDies;
  const int t = (2 * j + 1) * die_cost(x);
  int pos = 0;
#pragma unroll
  for (int y = 0; y < kDies; ++y) {
    const int c = die_cost(y);
    int cnt = ((t - 1) / c + 1) / 2;                     // j' with (2j' + 1) c < t
    if (y < x && t % c == 0 && ((t / c) & 1)) ++cnt;     // the same time, lower die
    pos += min(cnt, n);
  }
  return pos;
}

// ---------------------------------------------------------------------------
// Fused append: the new token of a decode step.

// 16-bit input element -> fp32 (exact).
template <typename IT>
__device__ __forceinline__ float in_value(uint16_t bits) {
  if constexpr (__is_same(IT, F16)) return (float)__builtin_bit_cast(_Float16, bits);
  else return __builtin_bit_cast(float, (uint32_t)bits << 16);
}
// Low / high 16-bit input element of a packed pair -> fp32 (exact).
template <typename IT>
__device__ __forceinline__ float in_lo(uint32_t w) {
  if constexpr (__is_same(IT, F16)) return f16_lo(w);
  else return bf16_lo(w);
}
template <typename IT>
__device__ __forceinline__ float in_hi(uint32_t w) {
  if constexpr (__is_same(IT, F16)) return f16_hi(w);
  else return bf16_hi(w);
}

// Row of sequence s, kv head kvh, in the new tokens' K or V input.
__device__ __forceinline__ const uint16_t* new_token_row(const DecodeParams& p, const void* base,
                                                         int s, int kvh, int D) {
  return reinterpret_cast<const uint16_t*>(base) + (int64_t)s * p.kv_token_stride +
         (int64_t)kvh * D;
}

// The new token of sequence s, kv head kvh, spread over one wavefront: lane
// l holds dims l, l + 64, ... of its K and V input rows.  Used in three
// steps: load (issued before the wavefront's first tile loads, so waiting
// for it does not wait for them), stage (the values the cache will hold, into
// LDS, from registers), write (the stores into the cache slot, issued after
// the wavefront's tile stream: vector loads and stores share one in-order
// counter on this target, so an early store would hold back the waits for
// every tile loaded after it).
template <int D>
struct NewToken {
  static constexpr int N = D / kWave;
  uint16_t k[N];
  uint16_t v[N];

  __device__ __forceinline__ void load(const DecodeParams& p, int s, int kvh, int lane) {
    const uint16_t* kin = new_token_row(p, p.k_new, s, kvh, D);
    const uint16_t* vin = new_token_row(p, p.v_new, s, kvh, D);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      k[i] = kin[lane + kWave * i];
      v[i] = vin[lane + kWave * i];
    }
  }

  // The values the cache holds for the token (code units, fp32) into LDS,
  // s_kv[d] for K and s_kv[D + d] for V, and what write() stores (the input
  // bits, or the fp8 codes) into s_bits[d] / s_bits[D + d], so that no
  // register holds the token through the stream.
  template <typename IT, typename CT>
  __device__ __forceinline__ void stage(const DecodeParams& p, int lane, float* s_kv,
                                        uint16_t* s_bits) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int d = lane + kWave * i;
      if constexpr (CT::kBytes == 2) {
        s_kv[d] = in_value<IT>(k[i]);
        s_kv[D + d] = in_value<IT>(v[i]);
        s_bits[d] = k[i];
        s_bits[D + d] = v[i];
      } else {
        const uint32_t kq = e4m3fn_encode(in_value<IT>(k[i]) * p.k_inv_scale);
        const uint32_t vq = e4m3fn_encode(in_value<IT>(v[i]) * p.v_inv_scale);
        s_kv[d] = fp8x2_to_f32<false>(kq)[0];
        s_kv[D + d] = fp8x2_to_f32<false>(vq)[0];
        s_bits[d] = (uint16_t)kq;
        s_bits[D + d] = (uint16_t)vq;
      }
    }
  }

  // Store the token at its slot (K row of the token-major tile; V dims at
  // (t/4*D + d)*4 + t%4 of the quad tile) exactly as the cache write does,
  // from what stage() left in s_bits; a negative slot or one past the pool
  // stores nothing.
  template <typename CT, int BS>
  static __device__ __forceinline__ void write(const DecodeParams& p, int32_t slot, int kvh,
                                               int lane, const uint16_t* s_bits) {
    const int64_t blk = slot / BS;
    const int off = slot % BS;
    if (slot < 0 || blk >= p.num_blocks) return;
    const int64_t tile = (blk * p.num_kv_heads + kvh) * (int64_t)(BS * D);   // elements
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int d = lane + kWave * i;
      const int64_t ko = tile + (int64_t)off * D + d;
      const int64_t vo = tile + ((int64_t)(off >> 2) * D + d) * 4 + (off & 3);
      if constexpr (CT::kBytes == 2) {
        reinterpret_cast<uint16_t*>(const_cast<void*>(p.k_cache))[ko] = s_bits[d];
        reinterpret_cast<uint16_t*>(const_cast<void*>(p.v_cache))[vo] = s_bits[D + d];
      } else {
        reinterpret_cast<uint8_t*>(const_cast<void*>(p.k_cache))[ko] = (uint8_t)s_bits[d];
        reinterpret_cast<uint8_t*>(const_cast<void*>(p.v_cache))[vo] = (uint8_t)s_bits[D + d];
      }
    }
  }
};

}  // namespace pa
