// Random-operation stress of the host block allocator through its C ABI, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by test_alloc_sanitized.py.
// Checks after every operation: every block is either free or referenced,
// counts equal table occurrences, the last block of a table has room for
// context_len; at the end, freeing everything returns every block.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

static int check(pa_allocator* a, const std::vector<int64_t>& live, int N, int B) {
  std::vector<int> occ(N, 0), fr(N, 0);
  std::vector<int32_t> fl(N > 0 ? N : 1);
  int nf = pa_alloc_free_list(a, fl.data(), N);
  for (int i = 0; i < nf; ++i) {
    if (fl[i] < 0 || fl[i] >= N || fr[fl[i]]++) return 1;
  }
  for (int64_t s : live) {
    int nb = pa_alloc_num_table_blocks(a, s);
    int ctx = pa_alloc_context_len(a, s);
    if (nb < 0 || ctx < 0) return 2;
    if (nb * B - ctx < 0 || nb * B - ctx > B - 1) { if (!(nb == 0 && ctx == 0)) return 3; }
    std::vector<int32_t> t(nb > 0 ? nb : 1);
    if (pa_alloc_block_tables(a, &s, 1, nb, t.data(), nullptr) != PA_OK) return 4;
    for (int j = 0; j < nb; ++j) occ[t[j]]++;
  }
  for (int b = 0; b < N; ++b) {
    if (pa_alloc_ref_count(a, b) != occ[b]) return 5;
    if ((occ[b] > 0) == (fr[b] > 0)) return 6;
  }
  return 0;
}

int main() {
  std::mt19937_64 rng(12345);
  for (int round = 0; round < 300; ++round) {
    const int N = static_cast<int>(rng() % 40);
    const int B = 1 << (rng() % 5);
    std::vector<int32_t> order(N);
    for (int i = 0; i < N; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pa_allocator* a = nullptr;
    if (pa_alloc_create(N, B, N ? order.data() : nullptr, &a) != PA_OK) return 10;
    std::vector<int64_t> live;
    for (int step = 0; step < 200; ++step) {
      const int kind = static_cast<int>(rng() % 4);
      const int64_t x = static_cast<int64_t>(rng() % 10);
      if (kind == 0) {
        if (pa_alloc_add_seq(a, x, static_cast<int32_t>(rng() % 50)) == PA_OK) live.push_back(x);
      } else if (kind == 1) {
        const int64_t y = static_cast<int64_t>(rng() % 10);
        if (pa_alloc_fork(a, x, y) == PA_OK) live.push_back(y);
      } else if (kind == 2 && !live.empty()) {
        std::vector<int64_t> ids(live.begin(), live.begin() + 1 + rng() % live.size());
        std::vector<int64_t> slots(ids.size()), pairs(2 * ids.size());
        int32_t ncow = 0;
        int rc = pa_alloc_append_slots(a, ids.data(), static_cast<int32_t>(ids.size()), slots.data(), pairs.data(),
                                       static_cast<int32_t>(ids.size()), &ncow);
        if (rc != PA_OK && rc != PA_ERR_NO_BLOCKS) return 11;
        for (size_t i = 0; rc == PA_OK && i < ids.size(); ++i)
          if (slots[i] < 0 || slots[i] >= static_cast<int64_t>(N) * B) return 12;
      } else if (kind == 3 && !live.empty()) {
        size_t k = rng() % live.size();
        if (pa_alloc_free_seq(a, live[k]) != PA_OK) return 13;
        live.erase(live.begin() + k);
      }
      int c = check(a, live, N, B);
      if (c) { std::printf("invariant %d broken at round %d step %d\n", c, round, step); return 20 + c; }
    }
    for (int64_t s : live) pa_alloc_free_seq(a, s);
    if (pa_alloc_num_free(a) != N) return 30;
    pa_alloc_destroy(a);
  }
  std::printf("ok\n");
  return 0;
}
