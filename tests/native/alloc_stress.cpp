// Random-operation stress of the host block allocator through its C ABI, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by test_alloc_sanitized.py.
// Half of the rounds turn prefix caching on; every round has a swap space.
// Checks after every operation: every block is either free or referenced,
// counts equal occurrences in resident tables, the last block of a table has
// room for context_len, every swap block is free or in exactly one swapped-out
// table, and the cached-block count matches the per-block flags; at the end,
// freeing everything returns every block of both pools.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

static int check(pa_allocator* a, const std::vector<int64_t>& live, int N, int B, int S) {
  std::vector<int> occ(N, 0), fr(N, 0), socc(S, 0);
  std::vector<int32_t> fl(N > 0 ? N : 1), sfl(S > 0 ? S : 1);
  int nf = pa_alloc_free_list(a, fl.data(), N);
  for (int i = 0; i < nf; ++i) {
    if (fl[i] < 0 || fl[i] >= N || fr[fl[i]]++) return 1;
  }
  int nsf = pa_alloc_swap_free_list(a, sfl.data(), S);
  for (int i = 0; i < nsf; ++i) {
    if (sfl[i] < 0 || sfl[i] >= S || socc[sfl[i]]++) return 7;
  }
  for (int64_t s : live) {
    int nb = pa_alloc_num_table_blocks(a, s);
    int ctx = pa_alloc_context_len(a, s);
    if (nb < 0 || ctx < 0) return 2;
    if (nb * B - ctx < 0 || nb * B - ctx > B - 1) { if (!(nb == 0 && ctx == 0)) return 3; }
    std::vector<int32_t> t(nb > 0 ? nb : 1);
    if (pa_alloc_seq_table(a, s, t.data(), nb) != nb) return 4;
    const int swapped = pa_alloc_is_swapped(a, s);
    for (int j = 0; j < nb; ++j) {
      if (swapped) {
        if (t[j] < 0 || t[j] >= S || socc[t[j]]++) return 8;
      } else {
        occ[t[j]]++;
      }
    }
  }
  int cached = 0;
  for (int b = 0; b < N; ++b) {
    if (pa_alloc_ref_count(a, b) != occ[b]) return 5;
    if ((occ[b] > 0) == (fr[b] > 0)) return 6;
    cached += pa_alloc_block_is_cached(a, b) == 1;
  }
  for (int b = 0; b < S; ++b)
    if (socc[b] != 1) return 9;
  if (pa_alloc_num_cached_blocks(a) != cached) return 10;
  return 0;
}

int main() {
  std::mt19937_64 rng(12345);
  const std::vector<std::vector<int32_t>> templates = {{1, 2, 3, 4, 5, 6, 7, 8}, {1, 2, 3, 4, 9, 9}, {7, 7, 7, 7}, {}};
  for (int round = 0; round < 300; ++round) {
    const int N = static_cast<int>(rng() % 40);
    const int B = 1 << (rng() % 5);
    const int S = static_cast<int>(rng() % 20);
    std::vector<int32_t> order(N);
    for (int i = 0; i < N; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pa_allocator* a = nullptr;
    if (pa_alloc_create(N, B, N ? order.data() : nullptr, &a) != PA_OK) return 10;
    if (pa_alloc_set_swap_space(a, S, nullptr) != PA_OK) return 14;
    if (round % 2 && pa_alloc_enable_prefix_caching(a) != PA_OK) return 15;
    std::vector<int64_t> live;
    for (int step = 0; step < 200; ++step) {
      const int kind = static_cast<int>(rng() % 9);
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
        if (rc != PA_OK && rc != PA_ERR_NO_BLOCKS && rc != PA_ERR_INVALID) return 11;
        for (size_t i = 0; rc == PA_OK && i < ids.size(); ++i)
          if (slots[i] < 0 || slots[i] >= static_cast<int64_t>(N) * B) return 12;
      } else if (kind == 3 && !live.empty()) {
        size_t k = rng() % live.size();
        if (pa_alloc_free_seq(a, live[k]) != PA_OK) return 13;
        live.erase(live.begin() + k);
      } else if (kind == 4 || kind == 7) {
        std::vector<int32_t> tok = templates[rng() % templates.size()];
        for (int t = static_cast<int>(rng() % 12); t > 0; --t) tok.push_back(static_cast<int32_t>(rng() % 3));
        const int64_t extra = static_cast<int64_t>(rng() % 2);
        if (kind == 4) {
          int32_t got = -1;
          int rc = pa_alloc_add_seq_cached(a, x, tok.empty() ? nullptr : tok.data(), static_cast<int32_t>(tok.size()),
                                           extra, &got);
          if (rc == PA_OK) {
            live.push_back(x);
            if (got < 0 || got % B || got > static_cast<int32_t>(tok.size())) return 16;
          }
        } else {
          std::vector<int32_t> hits(tok.size() + 1);
          int n = pa_alloc_prefix_hits(a, tok.empty() ? nullptr : tok.data(), static_cast<int32_t>(tok.size()), extra,
                                       hits.data(), static_cast<int32_t>(hits.size()));
          if (n < 0 || n > static_cast<int>(tok.size()) / B) return 17;
          for (int i = 0; i < n; ++i)
            if (pa_alloc_block_is_cached(a, hits[i]) != 1) return 18;
        }
      } else if ((kind == 5 || kind == 6) && !live.empty()) {
        const int64_t s = live[rng() % live.size()];
        const int nb = pa_alloc_num_table_blocks(a, s);
        std::vector<int64_t> pairs(2 * static_cast<size_t>(nb > 0 ? nb : 1));
        int32_t got = 0;
        int rc = kind == 5 ? pa_alloc_swap_out(a, s, pairs.data(), nb, &got) : pa_alloc_swap_in(a, s, pairs.data(), nb, &got);
        if (rc != PA_OK && rc != PA_ERR_NO_BLOCKS && rc != PA_ERR_INVALID) return 19;
        if (rc == PA_OK && got != nb) return 19;
      }
      if (kind == 8) {   // a batch of up to 3 prompts in one call
        const int nb = 1 + static_cast<int>(rng() % 3);
        std::vector<int64_t> ids(nb);
        std::vector<int32_t> lens(nb), tok;
        std::vector<int64_t> extra(nb);
        for (int i = 0; i < nb; ++i) {
          ids[i] = static_cast<int64_t>(rng() % 10);
          std::vector<int32_t> t = templates[rng() % templates.size()];
          for (int r = static_cast<int>(rng() % 12); r > 0; --r) t.push_back(static_cast<int32_t>(rng() % 3));
          lens[i] = static_cast<int32_t>(t.size());
          extra[i] = static_cast<int64_t>(rng() % 2);
          tok.insert(tok.end(), t.begin(), t.end());
        }
        std::vector<int64_t> slots(tok.size() + 1);
        std::vector<int32_t> cached(nb);
        int32_t admitted = -1;
        const bool use_tok = (round % 2) && !tok.empty();
        int rc = pa_alloc_admit(a, ids.data(), nb, use_tok ? tok.data() : nullptr, lens.data(), extra.data(),
                                slots.data(), cached.data(), &admitted);
        if (rc != PA_OK && rc != PA_ERR_NO_BLOCKS && rc != PA_ERR_INVALID) return 41;
        if (admitted < 0 || admitted > nb || (rc == PA_OK && admitted != nb)) return 42;
        for (int i = 0; i < admitted; ++i) live.push_back(ids[i]);
        for (size_t t = 0; t < tok.size(); ++t)
          if (slots[t] < -1 || slots[t] >= static_cast<int64_t>(N) * B) return 43;
      }
      int c = check(a, live, N, B, S);
      if (c) { std::printf("invariant %d broken at round %d step %d\n", c, round, step); return 20 + c; }
    }
    for (int64_t s : live) pa_alloc_free_seq(a, s);
    if (pa_alloc_num_free(a) != N || pa_alloc_num_free_swap(a) != S) return 40;
    pa_alloc_destroy(a);
  }
  std::printf("ok\n");
  return 0;
}
