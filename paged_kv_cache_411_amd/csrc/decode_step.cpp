// One decode step in one call: the host allocator's step, the launch schedule,
// and the copy-on-write copies, staged upload + append and attention launches
// on one stream. Plain C++17; the device work goes through the library's own
// launch entry points.
//
// Pages cited:
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//
// The order is that of a decode step ([PA] §3.3: allocate on demand, then
// write the new token's K/V; [VM] "写时复制与块共享机制": copy a shared block
// before it is written): slots and copy pairs from the allocator, the copies,
// the append (which also moves the staged tables, lengths and schedule to the
// device), then the attention over every listed sequence.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.h"
#include "pagedkv.h"
#include "status.h"

using pagedkv::fail;

namespace {

constexpr size_t kAlign = 256;
using pagedkv::kItemInts;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
size_t align16(size_t x) { return (x + 15) / 16 * 16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int pa_step_layout(int32_t num_seqs, int32_t width, int32_t block_size, int32_t partition_size,
                   pa_step_layout_t* out) {
  pagedkv::clear_error();
  if (out == nullptr || num_seqs < 0 || width < 1 || block_size <= 0 || partition_size < 0)
    return fail(PA_ERR_INVALID, "pa_step_layout: bad arguments");
  const int32_t max_part = pagedkv::kMaxPartitionBlocks * block_size;
  const int32_t part = pagedkv::effective_partition(partition_size, block_size);
  if (part > max_part || part % block_size != 0)
    return fail(PA_ERR_INVALID, "pa_step_layout: partition_size %d", partition_size);
  const int64_t n = num_seqs;
  // ranges per sequence: at most one more than its partitions (a shared run
  // and its own tokens may split one partition)
  const int64_t per_seq = (static_cast<int64_t>(width) * block_size + part - 1) / part + 1;
  const int64_t cap = n * per_seq;
  if (cap > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "pa_step_layout: %lld schedule items", (long long)cap);
  // Fixed-size regions first, then the schedule and the (padded) tables: the
  // step packs the tables right after the items it made and uploads only the
  // prefix that ends there.
  pa_step_layout_t L{};
  L.slots = 0;
  L.pairs = L.slots + align_up(8 * n);
  L.context_lens = L.pairs + align_up(16 * n);
  L.num_slots = L.context_lens + align_up(4 * n);
  L.members = L.num_slots + align_up(4 * n);
  L.work = L.members + align_up(4 * n);
  L.tables = L.work + align_up(static_cast<size_t>(4 * kItemInts) * cap);
  L.total = L.tables + align_up(4 * n * static_cast<size_t>(width));
  L.num_seqs = num_seqs;
  L.width = width;
  L.work_capacity = static_cast<int32_t>(cap);
  L.partition_size = part;
  *out = L;
  return PA_OK;
}

int pa_decode_step_plan(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, const pa_step_desc* d,
                        pa_step_plan_t* plan) {
  pagedkv::clear_error();
  if (a == nullptr || d == nullptr || plan == nullptr || n < 1 || seq_ids == nullptr || d->host_stage == nullptr ||
      !aligned16(d->host_stage))
    return fail(PA_ERR_INVALID, "pa_decode_step_plan: bad arguments (host_stage 16-byte aligned)");
  *plan = pa_step_plan_t{};
  const pa_step_layout_t& L = d->layout;
  const pa_cache_desc& c = d->cache;
  if (L.num_seqs != n) return fail(PA_ERR_INVALID, "pa_decode_step: layout is for %d sequences, %d given", L.num_seqs, n);
  if (L.total % 16 != 0 || L.work_capacity < 0 || c.block_size <= 0 ||
      static_cast<int64_t>(L.work_capacity) * c.num_kv_heads > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_decode_step: layout (total %zu, %d schedule items)", L.total, L.work_capacity);
  if (d->share_width < 1 || d->share_width > pa_decode_share_width())
    return fail(PA_ERR_INVALID, "pa_decode_step: share_width %d", d->share_width);
  char* h = static_cast<char*>(d->host_stage);
  int64_t* h_slots = reinterpret_cast<int64_t*>(h + L.slots);
  int64_t* h_pairs = reinterpret_cast<int64_t*>(h + L.pairs);
  int32_t* h_tables = reinterpret_cast<int32_t*>(h + L.tables);
  int32_t* h_ctx = reinterpret_cast<int32_t*>(h + L.context_lens);
  int32_t* h_work = reinterpret_cast<int32_t*>(h + L.work);
  int32_t* h_members = reinterpret_cast<int32_t*>(h + L.members);
  int32_t* h_nslots = reinterpret_cast<int32_t*>(h + L.num_slots);

  int32_t ncow = 0, max_ctx = 0;
  size_t upload = L.total;
  size_t tables_at = L.tables;
  int32_t entries = 0;
  int32_t nwork = 0, nmem = 0, max_slots = 0;
  if (!d->schedule) {
    // dense launch: padded tables
    int rc = pa_alloc_step(a, seq_ids, n, append, L.width, h_slots, h_pairs, n, &ncow, h_tables, h_ctx, &max_ctx);
    if (rc != PA_OK) return rc;   // nothing changed (a table longer than the layout's width included)
    max_ctx = std::max(max_ctx, 1);
  } else {
    // The allocator writes every table back to back at `tables` (each row the
    // sequence's whole table, ceil(ctx / B) entries); the schedule reads the
    // rows there; the packed rows then move down to right after the schedule
    // items it made (their destination lies at or below `tables`), and each
    // item names its sequence's row.
    thread_local std::vector<int32_t> starts, lens;
    thread_local std::vector<const int32_t*> rows;
    starts.resize(n);
    lens.resize(n);
    rows.resize(n);
    int rc = pagedkv::alloc_step_packed(a, seq_ids, n, append, L.width, h_slots, h_pairs, n, &ncow, h_tables,
                                        static_cast<int64_t>(n) * L.width, starts.data(), lens.data(), h_ctx,
                                        &max_ctx, &entries);
    if (rc != PA_OK) return rc;   // nothing changed (a table longer than the layout's width included)
    max_ctx = std::max(max_ctx, 1);
    for (int32_t i = 0; i < n; ++i) rows[i] = h_tables + starts[i];
    nwork = pagedkv::schedule_rows(h_ctx, rows.data(), lens.data(), n, c.block_size, L.partition_size, max_ctx,
                                   d->share_width, h_work, L.work_capacity, h_members, n, &nmem, h_nslots,
                                   &max_slots);
    if (nwork < 0)   // cannot happen with the layout's capacities
      return fail(PA_ERR_INVALID, "pa_decode_step: schedule failed after the allocator step: %s", pa_last_error());
    tables_at = L.work + align16(static_cast<size_t>(4 * kItemInts) * nwork);
    std::memmove(h + tables_at, h_tables, sizeof(int32_t) * static_cast<size_t>(entries));
    const int32_t B = c.block_size;
    for (int32_t k = 0; k < nwork; ++k) {
      int32_t* w = h_work + static_cast<size_t>(kItemInts) * k;
      const bool ok = w[0] >= 0 && w[0] < n;
      w[6] = ok ? starts[w[0]] : 0;
      w[7] = ok ? (h_ctx[w[0]] + B - 1) / B : 0;
    }
    upload = tables_at + align16(sizeof(int32_t) * static_cast<size_t>(entries));
  }
  plan->num_cow = ncow;
  plan->num_work = nwork;
  plan->num_members = nmem;
  plan->max_slots = max_slots;
  plan->max_context = max_ctx;
  plan->table_entries = entries;
  plan->tables_at = tables_at;
  plan->upload_bytes = upload;
  return PA_OK;
}

int pa_decode_step(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, const void* k_new,
                   const void* v_new, const void* q, void* out, void* k_cache, void* v_cache,
                   const pa_step_desc* d, void* stream, int32_t* out_max_context) {
  pagedkv::clear_error();
  if (out_max_context) *out_max_context = 0;
  if (a == nullptr || d == nullptr || n < 1 || seq_ids == nullptr || q == nullptr || out == nullptr ||
      k_cache == nullptr || v_cache == nullptr || d->host_stage == nullptr || d->dev_stage == nullptr ||
      (append && (k_new == nullptr || v_new == nullptr)))
    return fail(PA_ERR_INVALID, "pa_decode_step: bad arguments");
  const pa_step_layout_t& L = d->layout;
  const pa_cache_desc& c = d->cache;
  const bool fp8 = c.dtype == PA_FP8_E4M3 || c.dtype == PA_INT8;   // codes with a scale per row
  if (fp8 && (d->k_scale == nullptr || d->v_scale == nullptr))
    return fail(PA_ERR_INVALID, "pa_decode_step: an FP8 cache needs its scales");

  // Everything that can be refused is checked before the allocator moves:
  // every check the launches below make on their arguments is repeated here
  // (the host half, pa_decode_step_plan, checks its own before it steps).
  // q, out and the new rows have the cache's dtype, or f16 / bf16 over an FP8 cache.
  if (fp8 ? (d->q_dtype != PA_F16 && d->q_dtype != PA_BF16) : d->q_dtype != c.dtype)
    return fail(PA_ERR_INVALID, "pa_decode_step: q_dtype %d does not go with cache dtype %d", d->q_dtype, c.dtype);
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(d->host_stage) ||
      !aligned16(d->dev_stage) || (append && (!aligned16(k_new) || !aligned16(v_new))) ||
      (fp8 && (!aligned16(d->k_scale) || !aligned16(d->v_scale))))
    return fail(PA_ERR_INVALID, "pa_decode_step: q, out, caches, new rows, scales and stage buffers must be 16-byte aligned");
  if (!std::isfinite(d->scale)) return fail(PA_ERR_INVALID, "pa_decode_step: scale is not finite");
  if ((reinterpret_cast<uintptr_t>(d->done_flag) & 7u) != 0)
    return fail(PA_ERR_INVALID, "pa_decode_step: done_flag must be 8-byte aligned");
  pa_decode_desc dd{};
  dd.cache = c;
  dd.num_seqs = n;
  dd.num_q_heads = d->num_q_heads;
  dd.max_blocks_per_seq = L.width;
  dd.max_context_len = 0;   // bound: the table capacity
  dd.partition_size = L.partition_size;
  dd.q_dtype = d->q_dtype;
  const size_t need_ws = pa_decode_workspace_bytes(&dd, d->schedule != 0);
  if (need_ws == 0 && pa_last_error()[0] != '\0') return PA_ERR_INVALID;
  if (need_ws > d->workspace_bytes || (need_ws > 0 && (d->workspace == nullptr || !aligned16(d->workspace))))
    return fail(PA_ERR_INVALID, "pa_decode_step: a 16-byte aligned workspace of %zu bytes is needed (%zu given)",
                need_ws, d->workspace_bytes);

  pa_step_plan_t plan;
  int rc = pa_decode_step_plan(a, seq_ids, n, append, d, &plan);
  if (rc != PA_OK) return rc;   // nothing changed

  char* h = static_cast<char*>(d->host_stage);
  char* g = static_cast<char*>(d->dev_stage);
  const int64_t* h_slots = reinterpret_cast<const int64_t*>(h + L.slots);
  const int64_t* h_pairs = reinterpret_cast<const int64_t*>(h + L.pairs);
  if (plan.num_cow > 0) {
    rc = fp8 ? copy_blocks_fp8(k_cache, v_cache, d->k_scale, d->v_scale, h_pairs, plan.num_cow, &c, stream)
             : copy_blocks(k_cache, v_cache, h_pairs, plan.num_cow, &c, stream);
    if (rc != PA_OK) return rc;
  }
  // the last launch that reads host_stage; as it starts it stores done_value
  // into done_flag (every launch enqueued before it has then completed)
  if (append) {
    rc = fp8 ? pagedkv::append_fp8(k_new, v_new, d->q_dtype, h_slots, n, k_cache, v_cache, d->k_scale, d->v_scale,
                                   &c, g, h, plan.upload_bytes, stream, d->done_flag, d->done_value)
             : pagedkv::append_staged(k_new, v_new, h_slots, n, k_cache, v_cache, &c, g, h, plan.upload_bytes,
                                      stream, d->done_flag, d->done_value);
  } else {
    rc = pagedkv::stage_copy(g, h, plan.upload_bytes, stream, d->done_flag, d->done_value);
  }
  if (rc != PA_OK) return rc;

  dd.max_context_len = plan.max_context;
  dd.workspace = d->workspace;
  dd.workspace_bytes = d->workspace_bytes;
  dd.prof_events[0] = d->prof_events[0];
  dd.prof_events[1] = d->prof_events[1];
  if (d->schedule) {
    dd.work = reinterpret_cast<const int32_t*>(g + L.work);
    dd.num_work = plan.num_work;
    dd.members = plan.num_members > 0 ? reinterpret_cast<const int32_t*>(g + L.members) : nullptr;
    dd.num_members = plan.num_members;
    dd.num_slots = reinterpret_cast<const int32_t*>(g + L.num_slots);
    dd.max_slots = plan.max_slots;
    dd.compact_tables = 1;
    dd.table_entries = plan.table_entries;
  }
  if (fp8) {
    dd.k_scale = d->k_scale;
    dd.v_scale = d->v_scale;
  }
  rc = pa_decode(q, k_cache, v_cache, reinterpret_cast<const int32_t*>(g + plan.tables_at),
                 reinterpret_cast<const int32_t*>(g + L.context_lens), d->scale, out, &dd, stream);
  if (rc != PA_OK) return rc;
  if (out_max_context) *out_max_context = plan.max_context;
  return PA_OK;
}

}  // extern "C"
