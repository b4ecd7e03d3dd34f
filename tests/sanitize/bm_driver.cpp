// Standalone driver of the host block manager (pa_bm_*), built with
// AddressSanitizer and UndefinedBehaviorSanitizer (leak checking on at exit):
// seeded random traces of every call, with the manager's invariants checked
// after each step against a plain model kept here (who holds which block,
// how many free blocks each pool has).  Exit status 0 = clean; any sanitizer
// report aborts with a non-zero status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <iterator>
#include <map>
#include <vector>

#include "pa.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t rnd(uint32_t n) {   // xorshift64*, uniform enough for traces
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 2685821657736338717ull) >> 33) % (n ? n : 1);
}

int g_failures = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);  \
      ++g_failures;                                                 \
    }                                                               \
  } while (0)

// Every block's reference count equals the number of tables holding it, and
// free + referenced = pool size, in each pool.
void check_invariants(pa_block_manager* m, const std::map<int64_t, bool>& live, int32_t ngpu,
                      int32_t ncpu, int32_t bs) {
  std::vector<int32_t> cnt_gpu((size_t)ngpu, 0), cnt_cpu((size_t)ncpu, 0);
  for (auto& kv : live) {
    const int64_t len = pa_bm_seq_len(m, kv.first);
    CHECK(len >= 0);
    const int32_t nb = (int32_t)((len + bs - 1) / bs);
    std::vector<int32_t> row((size_t)(nb > 0 ? nb : 1));
    int64_t l2 = -1;
    CHECK(pa_bm_block_tables(m, &kv.first, 1, row.data(), nb, &l2) == PA_OK);
    CHECK(l2 == len);
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t b = row[(size_t)j];
      if (kv.second) {
        CHECK(b >= 0 && b < ngpu);
        if (b >= 0 && b < ngpu) ++cnt_gpu[(size_t)b];
      } else {
        CHECK(b >= 0 && b < ncpu);
        if (b >= 0 && b < ncpu) ++cnt_cpu[(size_t)b];
      }
    }
  }
  int32_t used_gpu = 0, used_cpu = 0;
  for (int32_t b = 0; b < ngpu; ++b) {
    CHECK(pa_bm_ref_count(m, b, 1) == cnt_gpu[(size_t)b]);
    used_gpu += cnt_gpu[(size_t)b] > 0;
  }
  for (int32_t b = 0; b < ncpu; ++b) {
    CHECK(pa_bm_ref_count(m, b, 0) == cnt_cpu[(size_t)b]);
    used_cpu += cnt_cpu[(size_t)b] > 0;
  }
  CHECK(pa_bm_num_free(m, 1) + used_gpu == ngpu);
  CHECK(pa_bm_num_free(m, 0) + used_cpu == ncpu);
}

void trace(uint64_t seed, int steps) {
  g_state = seed * 0x2545F4914F6CDD1Dull + 1;
  const int32_t bs = 1 + (int32_t)rnd(16);
  const int32_t ngpu = 1 + (int32_t)rnd(96), ncpu = (int32_t)rnd(64);
  std::vector<int32_t> order((size_t)ngpu);
  for (int32_t i = 0; i < ngpu; ++i) order[(size_t)i] = i;
  for (int32_t i = ngpu - 1; i > 0; --i) {
    const int32_t j = (int32_t)rnd((uint32_t)i + 1);
    const int32_t t = order[(size_t)i];
    order[(size_t)i] = order[(size_t)j];
    order[(size_t)j] = t;
  }
  pa_block_manager* m = pa_bm_create(ngpu, ncpu, bs, rnd(2) ? order.data() : nullptr);
  CHECK(m != nullptr);
  if (!m) return;
  std::map<int64_t, bool> live;   // sequence -> on the GPU
  int64_t next_id = 0;
  for (int step = 0; step < steps; ++step) {
    const uint32_t op = rnd(9);
    const int64_t any = live.empty() ? next_id : std::next(live.begin(), rnd((uint32_t)live.size()))->first;
    if (op == 0 || live.empty()) {
      const int st = pa_bm_add_sequence(m, next_id, rnd(3 * bs + 1));
      if (st == PA_OK) live[next_id] = true;
      else CHECK(st == PA_ERR_NO_BLOCKS);
      ++next_id;
    } else if (op == 1) {
      const int st = pa_bm_fork(m, any, next_id);
      if (st == PA_OK) live[next_id] = true;
      else CHECK(st == PA_ERR_SEQUENCE && !live[any]);
      ++next_id;
    } else if (op == 2 || op == 3) {
      int32_t slot = -2, pair[2] = {-2, -2};
      const int st = pa_bm_append_slot(m, any, &slot, pair);
      CHECK(st == PA_OK || st == PA_ERR_NO_BLOCKS || st == PA_ERR_SEQUENCE);
      if (st == PA_OK) CHECK(slot >= 0 && slot < ngpu * bs);
    } else if (op == 4) {
      // a batch of distinct sequences (a decode step), sometimes with a duplicate
      std::vector<int64_t> ids;
      for (auto& kv : live)
        if (rnd(2)) ids.push_back(kv.first);
      if (!ids.empty() && rnd(8) == 0) ids.push_back(ids[0]);
      std::vector<int32_t> slots(ids.size() + 1), pairs(2 * ids.size() + 2);
      int32_t nc = -1;
      const int st = pa_bm_append_slots(m, ids.data(), (int32_t)ids.size(), slots.data(),
                                        pairs.data(), &nc);
      CHECK(st == PA_OK || st == PA_ERR_NO_BLOCKS || st == PA_ERR_SEQUENCE);
      if (st == PA_OK) CHECK(nc >= 0 && nc <= (int32_t)ids.size());
    } else if (op == 5) {
      if (pa_bm_free(m, any) == PA_OK) live.erase(any);
    } else if (op == 6 || op == 7) {
      const int64_t len = pa_bm_seq_len(m, any);
      const int32_t k = (int32_t)((len + bs - 1) / bs);
      std::vector<int32_t> pairs((size_t)(2 * (k + 1)));
      int32_t np = -1;
      const bool out = live[any];
      const int st = out ? pa_bm_swap_out(m, any, pairs.data(), k, &np)
                         : pa_bm_swap_in(m, any, pairs.data(), k, &np);
      CHECK(st == PA_OK || st == PA_ERR_NO_BLOCKS);
      if (st == PA_OK) {
        CHECK(np == k);
        live[any] = !out;
      }
      if (k > 0) CHECK(pa_bm_swap_out(m, any, pairs.data(), k - 1, &np) != PA_OK);
    } else {
      // calls that must be refused and change nothing
      int32_t slot, pair[2];
      CHECK(pa_bm_append_slot(m, next_id + 1000, &slot, pair) == PA_ERR_SEQUENCE);
      CHECK(pa_bm_add_sequence(m, any, 1) == PA_ERR_SEQUENCE);
      CHECK(pa_bm_add_sequence(m, next_id + 1000, -1) == PA_ERR_SHAPE);
      CHECK(pa_bm_free(m, next_id + 1000) == PA_ERR_SEQUENCE);
      CHECK(pa_bm_block_tables(m, &any, 1, nullptr, 0, nullptr) == PA_ERR_NULL);
    }
    check_invariants(m, live, ngpu, ncpu, bs);
  }
  pa_bm_destroy(m);
}

}  // namespace

int main(int argc, char** argv) {
  const int traces = argc > 1 ? atoi(argv[1]) : 200;
  // invalid managers
  CHECK(pa_bm_create(-1, 0, 16, nullptr) == nullptr);
  CHECK(pa_bm_create(4, 0, 0, nullptr) == nullptr);
  const int32_t dup[3] = {0, 1, 1};
  CHECK(pa_bm_create(3, 0, 16, dup) == nullptr);
  CHECK(pa_bm_create(INT32_MAX, 0, 16, nullptr) == nullptr);
  for (int t = 0; t < traces; ++t) trace((uint64_t)t + 1, 300);
  printf("bm_sanitize: %d traces, %d failed checks\n", traces, g_failures);
  return g_failures == 0 ? 0 : 1;
}
