// Host-side physical block allocator: FIFO free queue, reference counts and
// per-sequence block tables, with fork, on-demand growth, copy-on-write and
// release. Plain C++17 with no HIP dependency.
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//   [KVM] "深入解析 vLLM 的 KV Cache 管理器：从内存碎片到 PagedAttention 的完整技术剖析"
//
// Every operation is O(1) per block it touches ([PA] §3.1: O(1) allocate and
// free): the free queue is a ring buffer of num_blocks entries, counts are a
// flat array, and a sequence's table is a vector of physical ids.

#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pagedkv::fail;

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  double watermark = 0.0;

  // FIFO free queue ([VM] "Python 演示": pop(0) / append; [KVM] Part 4: BlockPool
  // allocate() pops the head). ring[(head + i) % num_blocks], i < free_count.
  std::vector<int32_t> ring;
  int32_t head = 0;
  int32_t free_count = 0;

  std::vector<int32_t> ref;  // reference count per physical block

  struct Seq {
    std::vector<int32_t> table;  // logical block j -> physical id ([PA] §3.2)
    int32_t context_len = 0;
    bool swapped = false;        // table holds swap-space (host) block ids
  };
  std::unordered_map<int64_t, Seq> seqs;

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

  int32_t take() {
    int32_t b = ring[head];
    head = (head + 1 == num_blocks) ? 0 : head + 1;
    --free_count;
    ref[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    int32_t tail = head + free_count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++free_count;
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
  a->ring.resize(num_blocks);
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
      a->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  }
  a->head = 0;
  a->free_count = num_blocks;
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
  std::unordered_map<int64_t, int> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "%s: unknown sequence %lld", who, (long long)seq_ids[i]);
    if (!seen.emplace(seq_ids[i], 1).second)
      return fail(PA_ERR_INVALID, "%s: sequence %lld listed twice", who, (long long)seq_ids[i]);
    if (it->second.swapped) return fail(PA_ERR_INVALID, "%s: sequence %lld is swapped out", who, (long long)seq_ids[i]);
    plan->list[i] = &it->second;
  }
  std::vector<int32_t> touched;
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
  AppendPlan plan;
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
  for (int32_t i = 0; i < n && out != nullptr; ++i) {
    int32_t k = a->head + i;
    if (k >= a->num_blocks) k -= a->num_blocks;
    out[i] = a->ring[k];
  }
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
