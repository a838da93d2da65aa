// Host-side physical block allocator: FIFO free queue, reference counts and
// per-sequence block tables, with fork, on-demand growth, copy-on-write,
// release, a swap pool and optional automatic prefix caching. Plain C++17 with
// no HIP dependency.
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//   [KVM] "深入解析 vLLM 的 KV Cache 管理器：从内存碎片到 PagedAttention 的完整技术剖析"
//
// Every operation is O(1) per block it touches ([PA] §3.1: O(1) allocate and
// free): the free queue is a doubly-linked list threaded through two arrays of
// num_blocks entries, so a block also leaves it from any position in O(1)
// ([KVM] Part 4 FreeKVCacheBlockQueue: a prefix-cache hit pulls a block out
// of the middle); counts are a flat array, and a sequence's table is a vector
// of physical ids.

#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "internal.h"
#include "pagedkv.h"
#include "status.h"

using pagedkv::fail;

namespace {

// Hash -> block map for the prefix cache: open addressing with linear
// probing over a power-of-two table at most half full (a block holds at most
// one entry), and backward-shift deletion, so lookups touch one or two
// adjacent slots and nothing is allocated after set-up. Hashes arrive
// already mixed, so their low bits pick the home slot.
struct BlockIndex {
  std::vector<uint64_t> keys;
  std::vector<int32_t> vals;   // -1 = empty
  uint64_t mask = 0;
  int32_t count = 0;

  void init(int32_t num_blocks) {
    uint64_t cap = 16;
    while (cap < 2 * static_cast<uint64_t>(num_blocks)) cap <<= 1;
    keys.assign(cap, 0);
    vals.assign(cap, -1);
    mask = cap - 1;
    count = 0;
  }
  int32_t find(uint64_t h) const {
    for (uint64_t i = h & mask;; i = (i + 1) & mask) {
      if (vals[i] < 0) return -1;
      if (keys[i] == h) return vals[i];
    }
  }
  void insert(uint64_t h, int32_t b) {   // h must not be present
    uint64_t i = h & mask;
    while (vals[i] >= 0) i = (i + 1) & mask;
    keys[i] = h;
    vals[i] = b;
    ++count;
  }
  void erase(uint64_t h) {
    uint64_t i = h & mask;
    while (vals[i] >= 0 && keys[i] != h) i = (i + 1) & mask;
    if (vals[i] < 0) return;
    // shift later members of the probe run back over the hole
    for (uint64_t j = (i + 1) & mask; vals[j] >= 0; j = (j + 1) & mask) {
      const uint64_t home = keys[j] & mask;
      // j's entry may fill the hole at i unless its home lies cyclically in (i, j]
      const bool stays = (i <= j) ? (home > i && home <= j) : (home > i || home <= j);
      if (stays) continue;
      keys[i] = keys[j];
      vals[i] = vals[j];
      i = j;
    }
    vals[i] = -1;
    --count;
  }
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  double watermark = 0.0;

  // FIFO free queue ([VM] "Python 演示": pop(0) / append; [KVM] Part 4: BlockPool
  // allocate() pops the head): nxt / prv link the free blocks, -1 ends the list.
  std::vector<int32_t> nxt, prv;
  int32_t head = -1, tail = -1;
  int32_t free_count = 0;

  // Automatic prefix caching ([KVM] Part 3 and Part 4). A full prompt block
  // is indexed by a chained 64-bit hash of (previous block's hash, extra key,
  // its tokens); the index maps a hash to one block, and each indexed block
  // keeps the parent hash, extra key and tokens it was indexed with, so a
  // lookup confirms the content and not just the hash.
  bool prefix_caching = false;
  BlockIndex index;
  std::vector<char> indexed;          // per block: holds an index entry
  std::vector<uint64_t> key_hash, key_parent;
  std::vector<int64_t> key_extra;
  std::vector<int32_t> key_tokens;    // [num_blocks][block_size]

  std::vector<int32_t> ref;  // reference count per physical block

  struct Seq {
    std::vector<int32_t> table;  // logical block j -> physical id ([PA] §3.2)
    int32_t context_len = 0;
    bool swapped = false;        // table holds swap-space (host) block ids
    uint64_t seen = 0;           // the last multi-sequence call that listed it (duplicate check)
  };
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t calls = 0;            // multi-sequence calls so far (stamps Seq::seen)

  // Swap space: host-side blocks that hold the KV of sequences moved out of
  // the GPU pool ([VM] "显存管理与调度策略设计": evicted to CPU memory and brought
  // back when the request is scheduled again). Also a FIFO queue.
  std::vector<int32_t> swap_ring;
  int32_t swap_head = 0;
  int32_t swap_free = 0;
  int32_t swap_take() {
    int32_t b = swap_ring[swap_head];
    swap_head = (swap_head + 1 == static_cast<int32_t>(swap_ring.size())) ? 0 : swap_head + 1;
    --swap_free;
    return b;
  }
  void swap_give_back(int32_t b) {
    int32_t tail = swap_head + swap_free;
    if (tail >= static_cast<int32_t>(swap_ring.size())) tail -= static_cast<int32_t>(swap_ring.size());
    swap_ring[tail] = b;
    ++swap_free;
  }

  // scratch for the all-or-nothing dry run of append_slots
  std::vector<int32_t> pending_dec;

  void unlink(int32_t b) {
    const int32_t p = prv[b], n = nxt[b];
    if (p >= 0) nxt[p] = n; else head = n;
    if (n >= 0) prv[n] = p; else tail = p;
    nxt[b] = prv[b] = -1;
    --free_count;
  }
  void give_back(int32_t b) {   // to the tail
    prv[b] = tail;
    nxt[b] = -1;
    if (tail >= 0) nxt[tail] = b; else head = b;
    tail = b;
    ++free_count;
  }
  void drop_index(int32_t b) {
    index.erase(key_hash[b]);
    indexed[b] = 0;
  }
  int32_t take() {              // from the head; an indexed block is evicted lazily here
    const int32_t b = head;
    unlink(b);
    if (prefix_caching && indexed[b]) drop_index(b);
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) give_back(b);
  }
};

extern "C" {

int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                    pa_allocator** out) {
  pagedkv::clear_error();
  if (out == nullptr) return fail(PA_ERR_INVALID, "pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID, "pa_alloc_create: num_blocks=%d block_size=%d", num_blocks, block_size);
  auto* a = new pa_allocator();
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->nxt.assign(num_blocks, -1);
  a->prv.assign(num_blocks, -1);
  a->ref.assign(num_blocks, 0);
  a->pending_dec.assign(num_blocks, 0);
  if (initial_free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return fail(PA_ERR_INVALID, "pa_alloc_create: initial order is not a permutation of 0..%d",
                    num_blocks - 1);
      }
      seen[b] = 1;
    }
  }
  for (int32_t i = 0; i < num_blocks; ++i) a->give_back(initial_free_order ? initial_free_order[i] : i);
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int pa_alloc_add_seq(pa_allocator* a, int64_t seq_id, int32_t num_tokens) {
  pagedkv::clear_error();
  if (a == nullptr) return fail(PA_ERR_INVALID, "pa_alloc_add_seq: NULL allocator");
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_alloc_add_seq: num_tokens=%d", num_tokens);
  if (a->seqs.count(seq_id)) return fail(PA_ERR_INVALID, "pa_alloc_add_seq: sequence %lld exists", (long long)seq_id);
  int64_t need = (static_cast<int64_t>(num_tokens) + a->block_size - 1) / a->block_size;
  if (need > a->free_count)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_add_seq: need %lld blocks, %d free", (long long)need, a->free_count);
  pa_allocator::Seq s;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(a->take());
  s.context_len = num_tokens;
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id) {
  pagedkv::clear_error();
  if (a == nullptr) return fail(PA_ERR_INVALID, "pa_alloc_fork: NULL allocator");
  auto p = a->seqs.find(parent_id);
  if (p == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_alloc_fork: unknown parent %lld", (long long)parent_id);
  if (p->second.swapped) return fail(PA_ERR_INVALID, "pa_alloc_fork: parent %lld is swapped out", (long long)parent_id);
  if (a->seqs.count(child_id)) return fail(PA_ERR_INVALID, "pa_alloc_fork: child %lld exists", (long long)child_id);
  pa_allocator::Seq c = p->second;  // same physical blocks, same length
  for (int32_t b : c.table) ++a->ref[b];
  a->seqs.emplace(child_id, std::move(c));
  return PA_OK;
}

}  // extern "C"

namespace {

// The sequences of an append call, resolved, plus what the call would take
// from the pool. Counts evolve along the list, so a block shared by k writers
// is copied by the first k-1 of them only ([KVM] Part 4 allocate_slots: count
// the new blocks, check the pool, then commit or give up).
struct AppendPlan {
  std::vector<pa_allocator::Seq*> list;
  int64_t need = 0;        // blocks taken from the queue
  int64_t copies = 0;      // copy-on-write pairs
  int32_t max_table = 0;   // longest table after the call
};

int plan_append(pa_allocator* a, const int64_t* seq_ids, int32_t n, bool append, const char* who,
                AppendPlan* plan) {
  const int32_t B = a->block_size;
  plan->list.resize(n);
  plan->need = plan->copies = 0;
  plan->max_table = 0;
  const uint64_t stamp = ++a->calls;   // a sequence listed twice meets its own stamp
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "%s: unknown sequence %lld", who, (long long)seq_ids[i]);
    if (it->second.seen == stamp)
      return fail(PA_ERR_INVALID, "%s: sequence %lld listed twice", who, (long long)seq_ids[i]);
    it->second.seen = stamp;
    if (it->second.swapped) return fail(PA_ERR_INVALID, "%s: sequence %lld is swapped out", who, (long long)seq_ids[i]);
    plan->list[i] = &it->second;
  }
  thread_local std::vector<int32_t> touched;
  touched.clear();
  for (int32_t i = 0; i < n; ++i) {
    const auto* s = plan->list[i];
    int32_t len = static_cast<int32_t>(s->table.size());
    if (append) {
      if (s->context_len % B == 0) {
        ++plan->need;
        ++len;
      } else {
        int32_t last = s->table.back();
        if (a->ref[last] - a->pending_dec[last] > 1) {
          ++plan->need;
          ++plan->copies;
          if (a->pending_dec[last]++ == 0) touched.push_back(last);
        }
      }
    }
    if (len > plan->max_table) plan->max_table = len;
  }
  for (int32_t b : touched) a->pending_dec[b] = 0;
  return PA_OK;
}

// Commit a planned append ([PA] §3.3 steps 1-3; [VM] "写时复制与块共享机制").
int32_t commit_append(pa_allocator* a, const AppendPlan& plan, int64_t* out_slots, int64_t* out_cow_pairs) {
  const int32_t B = a->block_size;
  int32_t ncow = 0;
  for (size_t i = 0; i < plan.list.size(); ++i) {
    auto* s = plan.list[i];
    const int32_t pos = s->context_len;
    if (pos % B == 0) {
      s->table.push_back(a->take());
    } else {
      int32_t last = s->table.back();
      if (a->ref[last] > 1) {
        int32_t fresh = a->take();
        out_cow_pairs[2 * ncow] = last;
        out_cow_pairs[2 * ncow + 1] = fresh;
        ++ncow;
        --a->ref[last];
        s->table.back() = fresh;
      }
    }
    out_slots[i] = static_cast<int64_t>(s->table[pos / B]) * B + pos % B;
    s->context_len = pos + 1;
  }
  return ncow;
}

void write_tables(const AppendPlan& plan, int32_t max_blocks, int32_t* out_tables, int32_t* out_context_lens,
                  int32_t* out_max_context) {
  int32_t mc = 0;
  for (size_t i = 0; i < plan.list.size(); ++i) {
    const auto* s = plan.list[i];
    const auto& t = s->table;
    if (out_tables) {
      int32_t* row = out_tables + static_cast<int64_t>(i) * max_blocks;
      if (!t.empty()) std::memcpy(row, t.data(), t.size() * sizeof(int32_t));
      for (int32_t j = static_cast<int32_t>(t.size()); j < max_blocks; ++j) row[j] = -1;
    }
    if (out_context_lens) out_context_lens[i] = s->context_len;
    if (s->context_len > mc) mc = s->context_len;
  }
  if (out_max_context) *out_max_context = mc;
}

}  // namespace

extern "C" {

int pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n, int64_t* out_slots,
                          int64_t* out_cow_pairs, int32_t cow_capacity, int32_t* out_num_cow) {
  pagedkv::clear_error();
  if (a == nullptr || (n > 0 && (seq_ids == nullptr || out_slots == nullptr)) || n < 0)
    return fail(PA_ERR_INVALID, "pa_alloc_append_slots: bad arguments");
  if (out_num_cow) *out_num_cow = 0;
  AppendPlan plan;
  int rc = plan_append(a, seq_ids, n, true, "pa_alloc_append_slots", &plan);
  if (rc != PA_OK) return rc;
  if (plan.need > a->free_count)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_append_slots: need %lld blocks, %d free", (long long)plan.need,
                a->free_count);
  if (plan.copies > 0 && (out_cow_pairs == nullptr || plan.copies > cow_capacity))
    return fail(PA_ERR_INVALID, "pa_alloc_append_slots: %lld copy pairs, capacity %d", (long long)plan.copies,
                cow_capacity);
  const int32_t ncow = commit_append(a, plan, out_slots, out_cow_pairs);
  if (out_num_cow) *out_num_cow = ncow;
  return PA_OK;
}

int32_t pa_alloc_table_width(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append) {
  pagedkv::clear_error();
  if (a == nullptr || n < 0 || (n > 0 && seq_ids == nullptr)) {
    fail(PA_ERR_INVALID, "pa_alloc_table_width: bad arguments");
    return -1;
  }
  AppendPlan plan;
  if (plan_append(a, seq_ids, n, append != 0, "pa_alloc_table_width", &plan) != PA_OK) return -1;
  return plan.max_table;
}

int pa_alloc_step(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, int32_t max_blocks,
                  int64_t* out_slots, int64_t* out_cow_pairs, int32_t cow_capacity, int32_t* out_num_cow,
                  int32_t* out_tables, int32_t* out_context_lens, int32_t* out_max_context) {
  pagedkv::clear_error();
  if (a == nullptr || n < 0 || max_blocks < 0 || (n > 0 && seq_ids == nullptr) ||
      (append && n > 0 && out_slots == nullptr))
    return fail(PA_ERR_INVALID, "pa_alloc_step: bad arguments");
  if (out_num_cow) *out_num_cow = 0;
  thread_local AppendPlan plan;
  int rc = plan_append(a, seq_ids, n, append != 0, "pa_alloc_step", &plan);
  if (rc != PA_OK) return rc;
  if (plan.max_table > max_blocks)
    return fail(PA_ERR_INVALID, "pa_alloc_step: a table needs %d blocks > %d", plan.max_table, max_blocks);
  if (plan.need > a->free_count)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_step: need %lld blocks, %d free", (long long)plan.need, a->free_count);
  if (plan.copies > 0 && (out_cow_pairs == nullptr || plan.copies > cow_capacity))
    return fail(PA_ERR_INVALID, "pa_alloc_step: %lld copy pairs, capacity %d", (long long)plan.copies, cow_capacity);
  if (append) {
    const int32_t ncow = commit_append(a, plan, out_slots, out_cow_pairs);
    if (out_num_cow) *out_num_cow = ncow;
  }
  write_tables(plan, max_blocks, out_tables, out_context_lens, out_max_context);
  return PA_OK;
}

}  // extern "C"

int pagedkv::alloc_step_packed(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append,
                               int32_t max_blocks, int64_t* out_slots, int64_t* out_cow_pairs, int32_t cow_capacity,
                               int32_t* out_num_cow, int32_t* out_packed, int64_t packed_capacity,
                               int32_t* out_starts, int32_t* out_lens, int32_t* out_context_lens,
                               int32_t* out_max_context, int32_t* out_entries) {
  pagedkv::clear_error();
  if (a == nullptr || n < 0 || max_blocks < 0 || (n > 0 && (seq_ids == nullptr || out_packed == nullptr ||
                                                            out_starts == nullptr || out_lens == nullptr)) ||
      (append && n > 0 && out_slots == nullptr))
    return fail(PA_ERR_INVALID, "pa_alloc_step: bad arguments");
  if (out_num_cow) *out_num_cow = 0;
  thread_local AppendPlan plan;
  int rc = plan_append(a, seq_ids, n, append != 0, "pa_alloc_step", &plan);
  if (rc != PA_OK) return rc;
  if (plan.max_table > max_blocks)
    return fail(PA_ERR_INVALID, "pa_alloc_step: a table needs %d blocks > %d", plan.max_table, max_blocks);
  if (static_cast<int64_t>(plan.max_table) * n > packed_capacity)
    return fail(PA_ERR_INVALID, "pa_alloc_step: packed tables may need %lld entries > %lld",
                (long long)plan.max_table * n, (long long)packed_capacity);
  if (plan.need > a->free_count)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_step: need %lld blocks, %d free", (long long)plan.need, a->free_count);
  if (plan.copies > 0 && (out_cow_pairs == nullptr || plan.copies > cow_capacity))
    return fail(PA_ERR_INVALID, "pa_alloc_step: %lld copy pairs, capacity %d", (long long)plan.copies, cow_capacity);
  if (append) {
    const int32_t ncow = commit_append(a, plan, out_slots, out_cow_pairs);
    if (out_num_cow) *out_num_cow = ncow;
  }
  int32_t mc = 0, at = 0;
  for (int32_t i = 0; i < n; ++i) {
    const auto* s = plan.list[i];
    const int32_t len = static_cast<int32_t>(s->table.size());
    if (len > 0) std::memcpy(out_packed + at, s->table.data(), len * sizeof(int32_t));
    out_starts[i] = at;
    out_lens[i] = len;
    at += len;
    if (out_context_lens) out_context_lens[i] = s->context_len;
    if (s->context_len > mc) mc = s->context_len;
  }
  if (out_max_context) *out_max_context = mc;
  if (out_entries) *out_entries = at;
  return PA_OK;
}

extern "C" {

int pa_alloc_free_seq(pa_allocator* a, int64_t seq_id) {
  pagedkv::clear_error();
  if (a == nullptr) return fail(PA_ERR_INVALID, "pa_alloc_free_seq: NULL allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_alloc_free_seq: unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped) {
    for (int32_t b : it->second.table) a->swap_give_back(b);   // ascending logical order
  } else {
    for (int32_t b : it->second.table) a->release(b);  // ascending logical order
  }
  a->seqs.erase(it);
  return PA_OK;
}

int pa_alloc_set_swap_space(pa_allocator* a, int32_t num_blocks, const int32_t* initial_free_order) {
  pagedkv::clear_error();
  if (a == nullptr || num_blocks < 0) return fail(PA_ERR_INVALID, "pa_alloc_set_swap_space: bad arguments");
  for (const auto& kv : a->seqs)
    if (kv.second.swapped) return fail(PA_ERR_INVALID, "pa_alloc_set_swap_space: a sequence is swapped out");
  std::vector<int32_t> ring(num_blocks);
  if (initial_free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return fail(PA_ERR_INVALID, "pa_alloc_set_swap_space: initial order is not a permutation of 0..%d",
                    num_blocks - 1);
      seen[b] = 1;
      ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) ring[i] = i;
  }
  a->swap_ring.swap(ring);
  a->swap_head = 0;
  a->swap_free = num_blocks;
  return PA_OK;
}

int pa_alloc_swap_out(pa_allocator* a, int64_t seq_id, int64_t* out_pairs, int32_t capacity, int32_t* out_num) {
  pagedkv::clear_error();
  if (out_num) *out_num = 0;
  if (a == nullptr || capacity < 0) return fail(PA_ERR_INVALID, "pa_alloc_swap_out: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_alloc_swap_out: unknown sequence %lld", (long long)seq_id);
  auto& sq = it->second;
  if (sq.swapped) return fail(PA_ERR_INVALID, "pa_alloc_swap_out: sequence %lld is already swapped out", (long long)seq_id);
  const int32_t n = static_cast<int32_t>(sq.table.size());
  if (n > a->swap_free)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_swap_out: need %d swap blocks, %d free", n, a->swap_free);
  if (n > 0 && (out_pairs == nullptr || n > capacity))
    return fail(PA_ERR_INVALID, "pa_alloc_swap_out: %d pairs, capacity %d", n, capacity);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t gpu = sq.table[j];
    const int32_t host = a->swap_take();
    out_pairs[2 * j] = gpu;        // copy GPU block -> swap block before the GPU block is reused
    out_pairs[2 * j + 1] = host;
    a->release(gpu);               // a block other sequences still share keeps its count - 1
    sq.table[j] = host;
  }
  sq.swapped = true;
  if (out_num) *out_num = n;
  return PA_OK;
}

int pa_alloc_swap_in(pa_allocator* a, int64_t seq_id, int64_t* out_pairs, int32_t capacity, int32_t* out_num) {
  pagedkv::clear_error();
  if (out_num) *out_num = 0;
  if (a == nullptr || capacity < 0) return fail(PA_ERR_INVALID, "pa_alloc_swap_in: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_alloc_swap_in: unknown sequence %lld", (long long)seq_id);
  auto& sq = it->second;
  if (!sq.swapped) return fail(PA_ERR_INVALID, "pa_alloc_swap_in: sequence %lld is not swapped out", (long long)seq_id);
  const int32_t n = static_cast<int32_t>(sq.table.size());
  if (n > a->free_count) return fail(PA_ERR_NO_BLOCKS, "pa_alloc_swap_in: need %d blocks, %d free", n, a->free_count);
  if (n > 0 && (out_pairs == nullptr || n > capacity))
    return fail(PA_ERR_INVALID, "pa_alloc_swap_in: %d pairs, capacity %d", n, capacity);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t host = sq.table[j];
    const int32_t gpu = a->take();
    out_pairs[2 * j] = host;       // copy swap block -> GPU block
    out_pairs[2 * j + 1] = gpu;
    a->swap_give_back(host);
    sq.table[j] = gpu;
  }
  sq.swapped = false;
  if (out_num) *out_num = n;
  return PA_OK;
}

int32_t pa_alloc_num_free_swap(const pa_allocator* a) { return a ? a->swap_free : -1; }

int32_t pa_alloc_swap_free_list(const pa_allocator* a, int32_t* out, int32_t cap) {
  if (a == nullptr) return -1;
  int32_t n = a->swap_free < cap ? a->swap_free : cap;
  for (int32_t i = 0; i < n && out != nullptr; ++i) {
    int32_t k = a->swap_head + i;
    if (k >= static_cast<int32_t>(a->swap_ring.size())) k -= static_cast<int32_t>(a->swap_ring.size());
    out[i] = a->swap_ring[k];
  }
  return a->swap_free;
}

int32_t pa_alloc_seq_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap) {
  if (a == nullptr) return -1;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return -1;
  const auto& t = it->second.table;
  const int32_t n = static_cast<int32_t>(t.size());
  for (int32_t j = 0; j < n && j < cap && out != nullptr; ++j) out[j] = t[j];
  return n;
}

int32_t pa_alloc_is_swapped(const pa_allocator* a, int64_t seq_id) {
  if (a == nullptr) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int pa_alloc_seq_slots(const pa_allocator* a, int64_t seq_id, int32_t start, int32_t count,
                       int64_t* out_slots) {
  pagedkv::clear_error();
  if (a == nullptr || (count > 0 && out_slots == nullptr) || start < 0 || count < 0)
    return fail(PA_ERR_INVALID, "pa_alloc_seq_slots: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_alloc_seq_slots: unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped) return fail(PA_ERR_INVALID, "pa_alloc_seq_slots: sequence %lld is swapped out", (long long)seq_id);
  const auto& t = it->second.table;
  const int32_t B = a->block_size;
  if (static_cast<int64_t>(start) + count > static_cast<int64_t>(t.size()) * B)
    return fail(PA_ERR_INVALID, "pa_alloc_seq_slots: positions past the sequence's blocks");
  for (int32_t i = 0; i < count; ++i) {
    int32_t p = start + i;
    out_slots[i] = static_cast<int64_t>(t[p / B]) * B + p % B;
  }
  return PA_OK;
}

int pa_alloc_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                          int32_t* out_tables, int32_t* out_context_lens) {
  pagedkv::clear_error();
  if (a == nullptr || n < 0 || max_blocks < 0 || (n > 0 && seq_ids == nullptr))
    return fail(PA_ERR_INVALID, "pa_alloc_block_tables: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PA_ERR_INVALID, "pa_alloc_block_tables: unknown sequence %lld", (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PA_ERR_INVALID, "pa_alloc_block_tables: sequence %lld is swapped out", (long long)seq_ids[i]);
    const auto& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > max_blocks)
      return fail(PA_ERR_INVALID, "pa_alloc_block_tables: sequence %lld has %zu blocks > %d",
                  (long long)seq_ids[i], t.size(), max_blocks);
    if (out_tables) {
      int32_t* row = out_tables + static_cast<int64_t>(i) * max_blocks;
      if (!t.empty()) std::memcpy(row, t.data(), t.size() * sizeof(int32_t));
      for (int32_t j = static_cast<int32_t>(t.size()); j < max_blocks; ++j) row[j] = -1;
    }
    if (out_context_lens) out_context_lens[i] = it->second.context_len;
  }
  return PA_OK;
}

int32_t pa_alloc_num_free(const pa_allocator* a) { return a ? a->free_count : -1; }
int32_t pa_alloc_num_blocks(const pa_allocator* a) { return a ? a->num_blocks : -1; }

int32_t pa_alloc_ref_count(const pa_allocator* a, int32_t block) {
  if (a == nullptr || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

int32_t pa_alloc_context_len(const pa_allocator* a, int64_t seq_id) {
  if (a == nullptr) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : it->second.context_len;
}

int32_t pa_alloc_num_table_blocks(const pa_allocator* a, int64_t seq_id) {
  if (a == nullptr) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : static_cast<int32_t>(it->second.table.size());
}

int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap) {
  if (a == nullptr) return -1;
  int32_t n = a->free_count < cap ? a->free_count : cap;
  int32_t b = a->head;
  for (int32_t i = 0; i < n && out != nullptr; ++i, b = a->nxt[b]) out[i] = b;
  return a->free_count;
}

int pa_alloc_set_watermark(pa_allocator* a, double fraction) {
  pagedkv::clear_error();
  if (a == nullptr || !(fraction >= 0.0 && fraction < 1.0))
    return fail(PA_ERR_INVALID, "pa_alloc_set_watermark: fraction must be in [0, 1)");
  a->watermark = fraction;
  return PA_OK;
}

int pa_alloc_can_allocate(const pa_allocator* a, int32_t num_blocks) {
  if (a == nullptr || num_blocks < 0) return 0;
  return static_cast<double>(a->free_count) - num_blocks >= a->watermark * a->num_blocks ? 1 : 0;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Automatic prefix caching ([KVM] Part 3 "APC 的工作机制" and "哈希链的设计";
// Part 4 BlockPool and allocate_slots)

namespace {

// Chained block hash. The block's tokens are hashed on their own - FNV-1a
// steps (64-bit offset basis and prime, applied to 32-bit words rather than
// bytes) in four interleaved lanes, folded with the same step - so the
// blocks of a prompt hash independently; the chain then links that value
// with the parent block's hash and the extra key through the splitmix64
// finaliser. The first block's parent hash is 0.
uint64_t fmix(uint64_t h) {
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}

uint64_t tokens_hash(const int32_t* tokens, int32_t n) {
  constexpr uint64_t kBasis = 14695981039346656037ull, kPrime = 1099511628211ull;
  uint64_t lane[4] = {kBasis, kBasis ^ 1, kBasis ^ 2, kBasis ^ 3};
  auto step = [](uint64_t h, uint32_t w) { return (h ^ w) * kPrime; };
  int32_t i = 0;
  for (; i + 4 <= n; i += 4)
    for (int l = 0; l < 4; ++l) lane[l] = step(lane[l], static_cast<uint32_t>(tokens[i + l]));
  for (int l = 0; i < n; ++i, ++l) lane[l] = step(lane[l], static_cast<uint32_t>(tokens[i]));
  uint64_t h = step(lane[0], static_cast<uint32_t>(n));
  for (int l = 1; l < 4; ++l) {
    h = step(h, static_cast<uint32_t>(lane[l]));
    h = step(h, static_cast<uint32_t>(lane[l] >> 32));
  }
  return h;
}

uint64_t chain_hash(uint64_t parent, int64_t extra, uint64_t block_tokens_hash) {
  return fmix(block_tokens_hash ^ fmix(parent + 0x9e3779b97f4a7c15ull * (static_cast<uint64_t>(extra) + 1)));
}

// Hashes of the prompt's full blocks (first block first) into *hashes, and
// the blocks of its longest indexed leading run into *hits. A block counts
// only when the index entry's parent hash, extra key and tokens all match.
void walk_prefix(const pa_allocator* a, const int32_t* tokens, int32_t n, int64_t extra,
                 std::vector<uint64_t>* hashes, std::vector<int32_t>* hits) {
  const int32_t B = a->block_size;
  const int32_t full = n / B;
  hashes->resize(full);
  hits->clear();
  uint64_t parent = 0;
  bool run = true;
  for (int32_t j = 0; j < full; ++j) (*hashes)[j] = tokens_hash(tokens + static_cast<int64_t>(j) * B, B);
  for (int32_t j = 0; j < full; ++j) {
    const int32_t* tok = tokens + static_cast<int64_t>(j) * B;
    const uint64_t h = chain_hash(parent, extra, (*hashes)[j]);
    (*hashes)[j] = h;
    if (run) {
      const int32_t b = a->index.find(h);
      run = false;
      if (b >= 0) {
        if (a->key_parent[b] == parent && a->key_extra[b] == extra &&
            std::memcmp(&a->key_tokens[static_cast<size_t>(b) * B], tok, sizeof(int32_t) * B) == 0) {
          hits->push_back(b);
          run = true;
        }
      }
    }
    parent = h;
  }
}

}  // namespace

extern "C" {

int pa_alloc_enable_prefix_caching(pa_allocator* a) {
  pagedkv::clear_error();
  if (a == nullptr) return fail(PA_ERR_INVALID, "pa_alloc_enable_prefix_caching: NULL allocator");
  if (!a->seqs.empty())
    return fail(PA_ERR_INVALID, "pa_alloc_enable_prefix_caching: enable it before any sequence exists");
  if (a->prefix_caching) return PA_OK;
  const size_t N = static_cast<size_t>(a->num_blocks);
  a->indexed.assign(N, 0);
  a->key_hash.assign(N, 0);
  a->key_parent.assign(N, 0);
  a->key_extra.assign(N, 0);
  a->key_tokens.assign(N * static_cast<size_t>(a->block_size), 0);
  a->index.init(a->num_blocks);
  a->prefix_caching = true;
  return PA_OK;
}

int pa_alloc_add_seq_cached(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                            int64_t extra_key, int32_t* out_cached_tokens) {
  pagedkv::clear_error();
  if (out_cached_tokens) *out_cached_tokens = 0;
  if (a == nullptr || num_tokens < 0 || (num_tokens > 0 && tokens == nullptr))
    return fail(PA_ERR_INVALID, "pa_alloc_add_seq_cached: bad arguments");
  if (!a->prefix_caching) return fail(PA_ERR_INVALID, "pa_alloc_add_seq_cached: prefix caching is off");
  if (a->seqs.count(seq_id))
    return fail(PA_ERR_INVALID, "pa_alloc_add_seq_cached: sequence %lld exists", (long long)seq_id);
  const int32_t B = a->block_size;
  std::vector<uint64_t> hashes;
  std::vector<int32_t> hits;
  walk_prefix(a, tokens, num_tokens, extra_key, &hashes, &hits);
  const int64_t total = (static_cast<int64_t>(num_tokens) + B - 1) / B;
  const int64_t need = total - static_cast<int64_t>(hits.size());
  int64_t idle = 0;  // hits that sit in the free queue
  for (int32_t b : hits) idle += a->ref[b] == 0;
  if (need > a->free_count - idle)
    return fail(PA_ERR_NO_BLOCKS, "pa_alloc_add_seq_cached: need %lld blocks, %lld free", (long long)need,
                (long long)(a->free_count - idle));
  pa_allocator::Seq s;
  s.table.reserve(total);
  for (int32_t b : hits) {
    if (a->ref[b] == 0) a->unlink(b);   // out of the free queue, from wherever it sits
    ++a->ref[b];
    s.table.push_back(b);
  }
  for (int64_t i = 0; i < need; ++i) s.table.push_back(a->take());
  for (size_t j = hits.size(); j < hashes.size(); ++j) {
    const uint64_t h = hashes[j];
    if (a->index.find(h) >= 0) continue;   // this content is already indexed at another block
    const int32_t b = s.table[j];
    a->index.insert(h, b);
    a->indexed[b] = 1;
    a->key_hash[b] = h;
    a->key_parent[b] = j ? hashes[j - 1] : 0;
    a->key_extra[b] = extra_key;
    std::memcpy(&a->key_tokens[static_cast<size_t>(b) * B], tokens + static_cast<int64_t>(j) * B,
                sizeof(int32_t) * B);
  }
  s.context_len = num_tokens;
  if (out_cached_tokens) *out_cached_tokens = static_cast<int32_t>(hits.size()) * B;
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int32_t pa_alloc_prefix_hits(const pa_allocator* a, const int32_t* tokens, int32_t num_tokens, int64_t extra_key,
                             int32_t* out_blocks, int32_t cap) {
  pagedkv::clear_error();
  if (a == nullptr || num_tokens < 0 || (num_tokens > 0 && tokens == nullptr)) {
    fail(PA_ERR_INVALID, "pa_alloc_prefix_hits: bad arguments");
    return -1;
  }
  if (!a->prefix_caching) return 0;
  std::vector<uint64_t> hashes;
  std::vector<int32_t> hits;
  walk_prefix(a, tokens, num_tokens, extra_key, &hashes, &hits);
  const int32_t n = static_cast<int32_t>(hits.size());
  for (int32_t i = 0; i < n && i < cap && out_blocks != nullptr; ++i) out_blocks[i] = hits[i];
  return n;
}

int32_t pa_alloc_num_cached_blocks(const pa_allocator* a) {
  return a == nullptr ? -1 : a->index.count;
}

int32_t pa_alloc_block_is_cached(const pa_allocator* a, int32_t block) {
  if (a == nullptr || block < 0 || block >= a->num_blocks) return -1;
  return a->prefix_caching && a->indexed[block] ? 1 : 0;
}

}  // extern "C"

extern "C" {

int pa_alloc_admit(pa_allocator* a, const int64_t* seq_ids, int32_t n, const int32_t* tokens,
                   const int32_t* lengths, const int64_t* extra_keys, int64_t* out_slots, int32_t* out_cached,
                   int32_t* out_admitted) {
  pagedkv::clear_error();
  if (out_admitted) *out_admitted = 0;
  if (a == nullptr || n < 0 || (n > 0 && (seq_ids == nullptr || lengths == nullptr || out_slots == nullptr)))
    return fail(PA_ERR_INVALID, "pa_alloc_admit: bad arguments");
  if (tokens != nullptr && !a->prefix_caching) return fail(PA_ERR_INVALID, "pa_alloc_admit: prefix caching is off");
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lengths[i] < 0) return fail(PA_ERR_INVALID, "pa_alloc_admit: lengths[%d] = %d", i, lengths[i]);
    total += lengths[i];
  }
  const int32_t B = a->block_size;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = lengths[i];
    int32_t cached = 0;
    const int rc = tokens != nullptr
                       ? pa_alloc_add_seq_cached(a, seq_ids[i], tokens + off, len, extra_keys ? extra_keys[i] : 0,
                                                 &cached)
                       : pa_alloc_add_seq(a, seq_ids[i], len);
    if (rc != PA_OK) {   // the ones before are admitted; the message names this one
      for (int64_t t = off; t < total; ++t) out_slots[t] = -1;
      return rc;
    }
    const auto& table = a->seqs.find(seq_ids[i])->second.table;
    int64_t* dst = out_slots + off;
    for (int32_t p = 0; p < cached; ++p) dst[p] = -1;
    for (int32_t j = cached / B, p0 = cached; p0 < len; ++j, p0 += B) {   // cached is a multiple of B
      const int64_t base = static_cast<int64_t>(table[j]) * B;
      const int32_t m = len - p0 < B ? len - p0 : B;
      for (int32_t q = 0; q < m; ++q) dst[p0 + q] = base + q;
    }
    if (out_cached) out_cached[i] = cached;
    if (out_admitted) *out_admitted = i + 1;
    off += len;
  }
  return PA_OK;
}

}  // extern "C"
