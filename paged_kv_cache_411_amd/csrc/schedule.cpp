// The launch schedule of pa_decode: which (sequence, token range) items the
// partition kernel runs, longest first, with the runs of whole blocks that
// several sequences share read once for all of them. Plain C++17 (host only).
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//
// [PA] §5.2 groups queries that reach the same physical blocks so that the
// blocks are read once for the group; [VM] "写时复制与块共享机制": forked beams
// and parallel samples hold their prompt's blocks in common. [PA] §3.2 batches
// requests with the same access pattern: the items run longest first.
//
// Everything here runs once per decode step on the host, so it avoids hash
// maps and per-call allocations: groups are found by sorting the sequences on
// their first block id, and the scratch vectors are reused across calls.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "internal.h"
#include "pagedkv.h"
#include "status.h"

namespace pagedkv {

int32_t schedule_rows(const int32_t* context_lens, const int32_t* const* rows, const int32_t* row_lens,
                      int32_t num_seqs, int32_t block_size, int32_t partition_size, int32_t max_context_len,
                      int32_t share_width, int32_t* out_work, int32_t capacity, int32_t* out_members,
                      int32_t member_capacity, int32_t* out_num_members, int32_t* out_num_slots,
                      int32_t* out_max_slots) {
  const int32_t part = effective_partition(partition_size, block_size);
  auto valid = [&](int32_t c) { return c > 0 && (max_context_len == 0 || c <= max_context_len); };
  auto full_blocks = [&](int32_t s) { return std::min(context_lens[s] / block_size, row_lens[s]); };

  // 1. Groups of up to share_width sequences whose tables start with the same
  //    physical blocks: sequences sorted by (first block id, sequence id), so
  //    each run of equal first blocks lists its sequences in ascending order;
  //    within a run the lowest sequence leads and takes the share_width - 1
  //    others with the longest common run of whole blocks.
  thread_local std::vector<int32_t> shared_blocks, group_of, by_first, rest, next, members;
  thread_local std::vector<std::pair<int32_t, int32_t>> cand;
  struct Group { int32_t leader, blocks, mbase, mcount; };
  thread_local std::vector<Group> groups;
  shared_blocks.assign(num_seqs, 0);
  group_of.assign(num_seqs, -1);
  by_first.clear();
  members.clear();
  groups.clear();
  if (share_width > 1) {
    // one 64-bit key per sequence, (first block id, sequence id), sign bit
    // flipped so that unsigned order is signed order: a plain integer sort
    thread_local std::vector<uint64_t> keys;
    keys.clear();
    for (int32_t s = 0; s < num_seqs; ++s)
      if (valid(context_lens[s]) && full_blocks(s) >= 1)
        keys.push_back((static_cast<uint64_t>(static_cast<uint32_t>(rows[s][0]) ^ 0x80000000u) << 32) |
                       static_cast<uint32_t>(s));
    std::sort(keys.begin(), keys.end());
    for (uint64_t k : keys) by_first.push_back(static_cast<int32_t>(k & 0xffffffffu));
    for (size_t r0 = 0; r0 < by_first.size();) {
      size_t r1 = r0 + 1;
      while (r1 < by_first.size() && rows[by_first[r1]][0] == rows[by_first[r0]][0]) ++r1;
      rest.assign(by_first.begin() + r0, by_first.begin() + r1);
      r0 = r1;
      while (rest.size() >= 2) {
        const int32_t lead = rest[0];
        const int32_t lead_full = full_blocks(lead);
        cand.clear();   // (common whole blocks, sequence)
        for (size_t i = 1; i < rest.size(); ++i) {
          const int32_t c = rest[i];
          const int32_t lim = std::min(lead_full, full_blocks(c));
          int32_t k = 0;
          while (k < lim && rows[c][k] == rows[lead][k]) ++k;
          if (k > 0) cand.push_back({k, c});
        }
        std::stable_sort(cand.begin(), cand.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
        if (cand.size() > static_cast<size_t>(share_width - 1)) cand.resize(share_width - 1);
        if (!cand.empty()) {
          const int32_t g = static_cast<int32_t>(groups.size());
          const int32_t mbase = static_cast<int32_t>(members.size());
          for (const auto& c : cand) members.push_back(c.second);
          std::sort(members.begin() + mbase, members.end());
          const int32_t blocks = cand.back().first;   // the run all of them share
          groups.push_back({lead, blocks, mbase, static_cast<int32_t>(cand.size())});
          group_of[lead] = g;
          shared_blocks[lead] = blocks;
          for (size_t i = mbase; i < members.size(); ++i) {
            group_of[members[i]] = g;
            shared_blocks[members[i]] = blocks;
          }
        }
        next.clear();
        for (size_t i = 1; i < rest.size(); ++i)
          if (group_of[rest[i]] < 0) next.push_back(rest[i]);
        rest.swap(next);
      }
    }
  }

  // 2. Each sequence's context is tiled into ranges of at most `part` tokens:
  //    first the shared run (one item per range for the whole group), then its
  //    own tokens. A range's slot is its position in the tiling.
  struct Item { int32_t len, s, t0, n, slot, mb, mc; };
  thread_local std::vector<Item> shared_items, own_items, empty_items;
  shared_items.clear();
  own_items.clear();
  empty_items.clear();
  int32_t max_slots = 0;
  auto cdiv = [](int32_t x, int32_t y) { return (x + y - 1) / y; };
  for (const Group& g : groups) {
    const int32_t len = g.blocks * block_size;
    for (int32_t t0 = 0, slot = 0; t0 < len; t0 += part, ++slot)
      shared_items.push_back({std::min(part, len - t0), g.leader, t0, std::min(part, len - t0), slot, g.mbase,
                              g.mcount});
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t c = context_lens[s];
    if (!valid(c)) {
      empty_items.push_back({0, s, 0, 0, 0, 0, 0});
      out_num_slots[s] = 1;
      max_slots = std::max(max_slots, 1);
      continue;
    }
    const int32_t sh = shared_blocks[s] * block_size;
    int32_t slot = cdiv(sh, part);
    for (int32_t t0 = sh; t0 < c; t0 += part, ++slot)
      own_items.push_back({std::min(part, c - t0), s, t0, std::min(part, c - t0), slot, 0, 0});
    out_num_slots[s] = slot;
    max_slots = std::max(max_slots, slot);
  }
  // 3. Longest first: shared items (their bytes serve several sequences), the
  //    other ranges by decreasing length, then the empty / out-of-range ones.
  //    Sorted on 64-bit keys (INT32_MAX - length, position): longer first,
  //    equal lengths in their order of creation, with no allocation.
  auto longest_first = [](std::vector<Item>& v) {
    thread_local std::vector<uint64_t> order;
    thread_local std::vector<Item> sorted;
    order.resize(v.size());
    for (size_t i = 0; i < v.size(); ++i)
      order[i] = (static_cast<uint64_t>(static_cast<uint32_t>(INT32_MAX - v[i].len)) << 32) | i;
    std::sort(order.begin(), order.end());
    sorted.resize(v.size());
    for (size_t i = 0; i < v.size(); ++i) sorted[i] = v[order[i] & 0xffffffffu];
    v.swap(sorted);
  };
  longest_first(shared_items);
  longest_first(own_items);
  const int64_t count = static_cast<int64_t>(shared_items.size()) + own_items.size() + empty_items.size();
  if (count > capacity || static_cast<int64_t>(members.size()) > member_capacity) {
    fail(PA_ERR_INVALID, "pa_decode_schedule: %lld items / %zu members, capacity %d / %d", (long long)count,
         members.size(), capacity, member_capacity);
    return -1;
  }
  int32_t n = 0;
  for (const auto* v : {&shared_items, &own_items, &empty_items})
    for (const Item& it : *v) {
      int32_t* o = out_work + static_cast<int64_t>(kItemInts) * n;
      o[0] = it.s;
      o[1] = it.t0;
      o[2] = it.n;
      o[3] = it.slot;
      o[4] = it.mb;
      o[5] = it.mc;
      o[6] = 0;
      o[7] = 0;
      ++n;
    }
  if (!members.empty()) std::copy(members.begin(), members.end(), out_members);
  if (out_num_members) *out_num_members = static_cast<int32_t>(members.size());
  if (out_max_slots) *out_max_slots = max_slots;
  return n;
}

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

int32_t pa_decode_share_width(void) { return kShareWidth; }

int32_t pa_decode_schedule(const int32_t* context_lens, const int32_t* block_tables, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                           int32_t max_context_len, int32_t share_width, int32_t* out_work, int32_t capacity,
                           int32_t* out_members, int32_t member_capacity, int32_t* out_num_members,
                           int32_t* out_num_slots, int32_t* out_max_slots) {
  clear_error();
  if (out_num_members) *out_num_members = 0;
  if (out_max_slots) *out_max_slots = 0;
  if ((num_seqs > 0 && (context_lens == nullptr || out_num_slots == nullptr)) || num_seqs < 0 || block_size <= 0 ||
      partition_size < 0 || max_context_len < 0 || capacity < 0 || (capacity > 0 && out_work == nullptr) ||
      share_width < 1 || share_width > kShareWidth ||
      (share_width > 1 && (block_tables == nullptr || max_blocks_per_seq <= 0)) || member_capacity < 0 ||
      (member_capacity > 0 && out_members == nullptr)) {
    fail(PA_ERR_INVALID, "pa_decode_schedule: bad arguments");
    return -1;
  }
  const int32_t part = effective_partition(partition_size, block_size);
  if (part > kMaxPartitionBlocks * block_size || part % block_size != 0) {
    fail(PA_ERR_INVALID, "pa_decode_schedule: partition_size %d", part);
    return -1;
  }
  thread_local std::vector<const int32_t*> rows;
  thread_local std::vector<int32_t> lens;
  rows.assign(num_seqs, nullptr);
  lens.assign(num_seqs, share_width > 1 ? max_blocks_per_seq : 0);
  if (share_width > 1)
    for (int32_t s = 0; s < num_seqs; ++s) rows[s] = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
  return schedule_rows(context_lens, rows.data(), lens.data(), num_seqs, block_size, partition_size,
                       max_context_len, share_width, out_work, capacity, out_members, member_capacity,
                       out_num_members, out_num_slots, out_max_slots);
}

}  // extern "C"
