// Internal: constants and host helpers shared by the library's sources (not
// part of the C ABI). Plain C++, no HIP.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pagedkv.h"

namespace pagedkv {

constexpr int kItemInts = 8;             // ints per launch-schedule item
constexpr int kShareWidth = 4;           // sequences one shared item serves (one query head per KV head)
constexpr int kDefaultPartition = 1024;  // tokens per partition when the caller gives 0
constexpr int kMaxPartitionBlocks = 64;  // a partition's block ids live in one 64-lane register

// The partition size a request of `partition_size` tokens gets (0 = the default).
inline int32_t effective_partition(int32_t partition_size, int32_t block_size) {
  const int32_t max_part = kMaxPartitionBlocks * block_size;
  return partition_size == 0 ? (kDefaultPartition < max_part ? kDefaultPartition : max_part) : partition_size;
}

// pa_decode_schedule over tables given as one row pointer per sequence
// (rows[s][j] for j < row_lens[s]); same outputs and errors.
int32_t schedule_rows(const int32_t* context_lens, const int32_t* const* rows, const int32_t* row_lens,
                      int32_t num_seqs, int32_t block_size, int32_t partition_size, int32_t max_context_len,
                      int32_t share_width, int32_t* out_work, int32_t capacity, int32_t* out_members,
                      int32_t member_capacity, int32_t* out_num_members, int32_t* out_num_slots,
                      int32_t* out_max_slots);

// pa_alloc_step with the tables written back to back instead of padded:
// the whole table of seq_ids[i] at out_packed + out_starts[i] (out_lens[i]
// entries, at most packed_capacity in all). Same checks, refusals (state
// unchanged) and other outputs as pa_alloc_step; *out_entries gets the total.
int alloc_step_packed(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, int32_t max_blocks,
                      int64_t* out_slots, int64_t* out_cow_pairs, int32_t cow_capacity, int32_t* out_num_cow,
                      int32_t* out_packed, int64_t packed_capacity, int32_t* out_starts, int32_t* out_lens,
                      int32_t* out_context_lens, int32_t* out_max_context, int32_t* out_entries);

// kv_append_staged, kv_append_fp8 and pa_stage_copy that also store
// done_value into the host word done_flag (when not NULL) as the kernel
// starts: pa_decode_step's progress word.
int append_staged(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                  void* v_cache, const pa_cache_desc* desc, void* stage_dst, const void* stage_src,
                  size_t stage_bytes, void* stream, uint64_t* done_flag, uint64_t done_value);
int append_fp8(const void* k, const void* v, int32_t src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
               void* k_cache, void* v_cache, float* k_scale, float* v_scale, const pa_cache_desc* desc,
               void* stage_dst, const void* stage_src, size_t stage_bytes, void* stream, uint64_t* done_flag,
               uint64_t done_value);
int stage_copy(void* dst, const void* src, size_t bytes, void* stream, uint64_t* done_flag, uint64_t done_value);

}  // namespace pagedkv
