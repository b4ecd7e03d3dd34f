// Host block manager of a paged KV cache (CPU code, no GPU calls).
//
// "How does paged attention work (in detail)", sections 2-4: the KV cache is
// a pool of fixed-size physical blocks and every sequence has a block table
// listing its logical blocks in order.  The manager hands out free blocks,
// counts references, returns a block to the free pool when its count drops
// to zero, gives a sequence that must write into a shared block its own copy
// (copy-on-write, section 3.3), maps a new block only when a token starts an
// unmapped logical block (section 4.1), and moves a preempted sequence's
// blocks to a CPU pool and back (section 4.3; the vLLM paper summary,
// section 5, names the CPU block allocator).
//
// Policy: free block ids wait in a FIFO queue; allocation takes from its
// front, freed blocks join its back in table order.  Every call either
// succeeds completely or changes nothing.  Not thread-safe: one caller at a
// time per manager.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

// FIFO of free block ids plus a reference count per block.
class Pool {
 public:
  bool init(int32_t n, const int32_t* order) {
    refs_.assign((size_t)n, 0);
    ring_.assign((size_t)(n > 0 ? n : 1), 0);
    head_ = 0;
    count_ = 0;
    std::vector<uint8_t> seen((size_t)n, 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = order ? order[i] : i;
      if (b < 0 || b >= n || seen[(size_t)b]) return false;
      seen[(size_t)b] = 1;
      push(b);
    }
    return true;
  }
  int32_t free_count() const { return count_; }
  int32_t ref(int32_t b) const {
    return (b >= 0 && (size_t)b < refs_.size()) ? refs_[(size_t)b] : 0;
  }
  // Take k blocks (caller checked free_count() >= k).
  void take(int32_t k, std::vector<int32_t>& out) {
    for (int32_t i = 0; i < k; ++i) {
      const int32_t b = ring_[(size_t)head_];
      head_ = (head_ + 1) % (int32_t)ring_.size();
      --count_;
      refs_[(size_t)b] = 1;
      out.push_back(b);
    }
  }
  void add_ref(int32_t b) { ++refs_[(size_t)b]; }
  void release(int32_t b) {
    if (--refs_[(size_t)b] == 0) push(b);
  }

 private:
  void push(int32_t b) {
    ring_[(size_t)((head_ + count_) % (int32_t)ring_.size())] = b;
    ++count_;
  }
  std::vector<int32_t> refs_;
  std::vector<int32_t> ring_;
  int32_t head_ = 0;
  int32_t count_ = 0;
};

struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
  bool on_gpu = true;
};

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

struct pa_block_manager {
  int32_t block_size = 0;
  Pool gpu;
  Pool cpu;
  std::unordered_map<int64_t, Seq> seqs;
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_gpu_blocks, int32_t num_cpu_blocks,
                               int32_t block_size, const int32_t* gpu_free_order) {
  if (num_gpu_blocks < 0 || num_cpu_blocks < 0 || block_size <= 0) return nullptr;
  // slots (block * block_size + offset) must fit the kernels' int32 slot_mapping
  if ((int64_t)num_gpu_blocks * block_size > INT32_MAX) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return nullptr;
  m->block_size = block_size;
  if (!m->gpu.init(num_gpu_blocks, gpu_free_order) || !m->cpu.init(num_cpu_blocks, nullptr)) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, int64_t num_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (m->seqs.count(seq_id)) return PA_ERR_SEQUENCE;
  const int64_t need = blocks_for(num_tokens, m->block_size);
  if (need > m->gpu.free_count()) return PA_ERR_NO_BLOCKS;
  Seq s;
  s.len = num_tokens;
  m->gpu.take((int32_t)need, s.blocks);
  m->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end() || !it->second.on_gpu || m->seqs.count(child)) return PA_ERR_SEQUENCE;
  Seq s = it->second;
  for (int32_t b : s.blocks) m->gpu.add_ref(b);
  m->seqs.emplace(child, std::move(s));
  return PA_OK;
}

int pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int32_t* slot, int32_t* copy_pair) {
  if (!m || !slot || !copy_pair) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || !it->second.on_gpu) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  const int32_t bs = m->block_size;
  const int64_t j = s.len / bs;
  copy_pair[0] = copy_pair[1] = -1;
  if (j == (int64_t)s.blocks.size()) {
    if (m->gpu.free_count() < 1) return PA_ERR_NO_BLOCKS;
    m->gpu.take(1, s.blocks);
  } else if (m->gpu.ref(s.blocks[(size_t)j]) > 1) {
    if (m->gpu.free_count() < 1) return PA_ERR_NO_BLOCKS;
    std::vector<int32_t> nb;
    m->gpu.take(1, nb);
    const int32_t old = s.blocks[(size_t)j];
    m->gpu.release(old);
    s.blocks[(size_t)j] = nb[0];
    copy_pair[0] = old;
    copy_pair[1] = nb[0];
  }
  *slot = s.blocks[(size_t)j] * bs + (int32_t)(s.len % bs);
  ++s.len;
  return PA_OK;
}

int pa_bm_append_slots(pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t* slots,
                       int32_t* copy_pairs, int32_t* num_copies) {
  if (!m || (n > 0 && (!seq_ids || !slots || !copy_pairs)) || !num_copies) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  // check first so that a failure changes nothing: every sequence known, on
  // the GPU and listed once, and enough free blocks (a copy-on-write earlier
  // in the batch can only lower the count needed later)
  int64_t need = 0;
  std::unordered_map<int64_t, int> listed;
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || !it->second.on_gpu || listed[seq_ids[i]]++) return PA_ERR_SEQUENCE;
    const Seq& s = it->second;
    const int64_t j = s.len / m->block_size;
    if (j == (int64_t)s.blocks.size() || m->gpu.ref(s.blocks[(size_t)j]) > 1) ++need;
  }
  if (need > m->gpu.free_count()) return PA_ERR_NO_BLOCKS;
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t pair[2];
    pa_bm_append_slot(m, seq_ids[i], &slots[i], pair);
    if (pair[0] >= 0) {
      copy_pairs[2 * nc] = pair[0];
      copy_pairs[2 * nc + 1] = pair[1];
      ++nc;
    }
  }
  *num_copies = nc;
  return PA_OK;
}

int pa_bm_free(pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  Pool& pool = it->second.on_gpu ? m->gpu : m->cpu;
  for (int32_t b : it->second.blocks) pool.release(b);
  m->seqs.erase(it);
  return PA_OK;
}

// Move a sequence between the pools; pairs [k][2] = (from, to) in table order.
static int move_seq(pa_block_manager* m, int64_t seq_id, bool to_cpu, int32_t* pairs,
                    int32_t max_pairs, int32_t* num_pairs) {
  if (!m || !num_pairs) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || it->second.on_gpu != to_cpu) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  const int32_t k = (int32_t)s.blocks.size();
  if (k > max_pairs || (k > 0 && !pairs)) return PA_ERR_SHAPE;
  Pool& from = to_cpu ? m->gpu : m->cpu;
  Pool& to = to_cpu ? m->cpu : m->gpu;
  if (k > to.free_count()) return PA_ERR_NO_BLOCKS;
  std::vector<int32_t> dst;
  to.take(k, dst);
  for (int32_t i = 0; i < k; ++i) {
    pairs[2 * i] = s.blocks[(size_t)i];
    pairs[2 * i + 1] = dst[(size_t)i];
    from.release(s.blocks[(size_t)i]);
  }
  s.blocks = std::move(dst);
  s.on_gpu = !to_cpu;
  *num_pairs = k;
  return PA_OK;
}

int pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int32_t* pairs, int32_t max_pairs,
                   int32_t* num_pairs) {
  return move_seq(m, seq_id, true, pairs, max_pairs, num_pairs);
}

int pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int32_t* pairs, int32_t max_pairs,
                  int32_t* num_pairs) {
  return move_seq(m, seq_id, false, pairs, max_pairs, num_pairs);
}

int pa_bm_block_tables(const pa_block_manager* m, const int64_t* seq_ids, int32_t n,
                       int32_t* tables, int32_t max_blocks, int64_t* lens) {
  if (!m || (n > 0 && (!seq_ids || !tables))) return PA_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
    if ((int64_t)it->second.blocks.size() > max_blocks) return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < (int32_t)s.blocks.size() ? s.blocks[(size_t)j] : -1;
    if (lens) lens[i] = s.len;
  }
  return PA_OK;
}

int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id) {
  if (!m) return -1;
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : it->second.len;
}

int32_t pa_bm_num_free(const pa_block_manager* m, int32_t on_gpu) {
  if (!m) return -1;
  return on_gpu ? m->gpu.free_count() : m->cpu.free_count();
}

int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block, int32_t on_gpu) {
  if (!m) return -1;
  return on_gpu ? m->gpu.ref(block) : m->cpu.ref(block);
}

}  // extern "C"
