// kv_append and copy_blocks for gfx950, and their C ABI entry points.
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//
// Both are byte moves: 16-byte vector loads and stores of raw bits, so the
// result is bit-exact for every dtype (NaN payloads and signed zeros kept).
//   kv_append   - [PA] §3.3 按需分配策略 step 4: a new token's K and V vectors go
//                 to its slot (block slot / B, offset slot % B) for every head.
//   copy_blocks - [VM] "写时复制与块共享机制" and [PA] §4.1: before a shared block
//                 is modified, its whole content (every head, every slot, K and
//                 V) is copied to the writer's new block.
// Ids and slots are range-checked on the device (out-of-range entries are
// skipped), so no input content can make these kernels touch memory outside
// the caches.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace pagedkv {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kCopyThreads = 256;
constexpr int kCopyVecsPerThread = 4;   // 16 KiB per workgroup

// All heads' rows of K and V of token i (row_vecs 16-byte vectors per head
// row), by one workgroup.
__device__ __forceinline__ void append_token(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                             const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
                                             uint4* __restrict__ v_cache, int num_kv_heads, int block_size,
                                             int row_vecs, int64_t num_slots, int64_t i) {
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int per_token = num_kv_heads * row_vecs;
  for (int idx = threadIdx.x; idx < per_token; idx += kAppendThreads) {
    const int h = idx / row_vecs;
    const int c = idx - h * row_vecs;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_vecs + c;
    const int64_t src = i * per_token + idx;
    const uint4 kk = k[src];
    const uint4 vv = v[src];
    k_cache[dst] = kk;
    v_cache[dst] = vv;
  }
}

// One workgroup per token.
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int num_kv_heads, int block_size, int row_vecs,
    int64_t num_slots) {
  append_token(k, v, slot_mapping, k_cache, v_cache, num_kv_heads, block_size, row_vecs, num_slots, blockIdx.x);
}

// kv_append and a staging copy in one launch: the first stage_wgs workgroups
// copy stage_n 16-byte vectors (grid-stride among themselves), the rest append
// one token each. The two parts touch disjoint memory.
__global__ __launch_bounds__(kAppendThreads) void kv_append_staged_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int num_kv_heads, int block_size, int row_vecs,
    int64_t num_slots, uint4* __restrict__ stage_dst, const uint4* __restrict__ stage_src, int64_t stage_n,
    int stage_wgs) {
  if (static_cast<int>(blockIdx.x) < stage_wgs) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAppendThreads + threadIdx.x; i < stage_n;
         i += static_cast<int64_t>(stage_wgs) * kAppendThreads)
      stage_dst[i] = stage_src[i];
    return;
  }
  append_token(k, v, slot_mapping, k_cache, v_cache, num_kv_heads, block_size, row_vecs, num_slots,
               static_cast<int64_t>(blockIdx.x) - stage_wgs);
}

// grid (slices of a block, pairs, 2 = K/V): each workgroup copies one 16 KiB
// slice of one block of one cache.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const int64_t* __restrict__ pairs,
    int64_t block_vecs, int64_t num_blocks) {
  const int64_t src = pairs[2 * static_cast<int64_t>(blockIdx.y)];
  const int64_t dst = pairs[2 * static_cast<int64_t>(blockIdx.y) + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* cache = blockIdx.z == 0 ? k_cache : v_cache;
  const uint4* from = cache + src * block_vecs;
  uint4* to = cache + dst * block_vecs;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyVecsPerThread + threadIdx.x;
  uint4 r[kCopyVecsPerThread];
#pragma unroll
  for (int j = 0; j < kCopyVecsPerThread; ++j) {
    const int64_t e = base + j * kCopyThreads;
    if (e < block_vecs) r[j] = from[e];
  }
#pragma unroll
  for (int j = 0; j < kCopyVecsPerThread; ++j) {
    const int64_t e = base + j * kCopyThreads;
    if (e < block_vecs) to[e] = r[j];
  }
}

// Plain 16-byte copy, grid-stride; src may be pinned host memory (read over
// the bus by the kernel itself).
__global__ __launch_bounds__(kCopyThreads) void stage_copy_kernel(uint4* __restrict__ dst,
                                                                 const uint4* __restrict__ src, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kCopyThreads)
    dst[i] = src[i];
}

int check_cache(const pa_cache_desc* c, const char* who) {
  if (c == nullptr) return fail(PA_ERR_INVALID, "%s: NULL desc", who);
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", who, c->dtype);
  const int eb = c->dtype == PA_F32 ? 4 : 2;
  if (c->num_blocks < 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_INVALID, "%s: blocks=%d kv_heads=%d block_size=%d head_dim=%d", who, c->num_blocks,
                c->num_kv_heads, c->block_size, c->head_dim);
  if ((static_cast<int64_t>(c->head_dim) * eb) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim * element bytes must be a multiple of 16", who);
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

namespace {

// Validation shared by kv_append and kv_append_staged (and the PA_DEBUG slot
// check); fills the row geometry.
int check_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                 void* v_cache, const pa_cache_desc* desc, hipStream_t stream, const char* who, int* row_vecs,
                 int64_t* num_slots) {
  int rc = check_cache(desc, who);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: num_tokens %d", who, num_tokens);
  const int eb = desc->dtype == PA_F32 ? 4 : 2;
  *row_vecs = desc->head_dim * eb / 16;
  *num_slots = static_cast<int64_t>(desc->num_blocks) * desc->block_size;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_INVALID, "%s: NULL pointer", who);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(PA_ERR_INVALID, "%s: k/v/caches must be 16-byte aligned", who);
  if (debug_enabled()) {
    std::vector<int64_t> s(num_tokens);
    if (hipMemcpyAsync(s.data(), slot_mapping, num_tokens * sizeof(int64_t), hipMemcpyDefault, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return fail(PA_ERR_HIP, "%s: debug copy failed", who);
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (s[i] < 0) continue;
      if (s[i] >= *num_slots)
        return fail(PA_ERR_INVALID, "%s: slot_mapping[%d] = %lld outside the pool", who, i, (long long)s[i]);
      if (!seen.insert(s[i]).second) return fail(PA_ERR_INVALID, "%s: slot %lld appears twice", who, (long long)s[i]);
    }
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
              void* v_cache, const pa_cache_desc* desc, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int row_vecs;
  int64_t num_slots;
  int rc = check_append(k, v, slot_mapping, num_tokens, k_cache, v_cache, desc, stream, "kv_append", &row_vecs,
                        &num_slots);
  if (rc != PA_OK || num_tokens == 0) return rc;
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_tokens), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), desc->num_kv_heads,
                     desc->block_size, row_vecs, num_slots);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_append: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int kv_append_staged(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                     void* v_cache, const pa_cache_desc* desc, void* stage_dst, const void* stage_src,
                     size_t stage_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int row_vecs;
  int64_t num_slots;
  int rc = check_append(k, v, slot_mapping, num_tokens, k_cache, v_cache, desc, stream, "kv_append_staged",
                        &row_vecs, &num_slots);
  if (rc != PA_OK) return rc;
  if (stage_bytes > 0 && (!stage_dst || !stage_src || !aligned16(stage_dst) || !aligned16(stage_src) ||
                          stage_bytes % 16 != 0))
    return fail(PA_ERR_INVALID, "kv_append_staged: staging pointers and size must be multiples of 16 bytes");
  const int64_t stage_n = static_cast<int64_t>(stage_bytes / 16);
  const int64_t want = (stage_n + kAppendThreads - 1) / kAppendThreads;
  const int stage_wgs = static_cast<int>(want < 256 ? want : 256);
  const int64_t grid = static_cast<int64_t>(stage_wgs) + num_tokens;
  if (grid == 0) return PA_OK;
  hipLaunchKernelGGL(kv_append_staged_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), desc->num_kv_heads,
                     desc->block_size, row_vecs, num_slots, static_cast<uint4*>(stage_dst),
                     static_cast<const uint4*>(stage_src), stage_n, stage_wgs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_append_staged: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int32_t num_pairs,
                const pa_cache_desc* desc, void* stream_) {
  clear_error();
  int rc = check_cache(desc, "copy_blocks");
  if (rc != PA_OK) return rc;
  if (num_pairs < 0 || num_pairs > 65535) return fail(PA_ERR_INVALID, "copy_blocks: num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return fail(PA_ERR_INVALID, "copy_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(src_dst_pairs) & 7u))
    return fail(PA_ERR_INVALID, "copy_blocks: caches must be 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (debug_enabled()) {
    std::vector<int64_t> pr(2 * static_cast<size_t>(num_pairs));
    if (hipMemcpyAsync(pr.data(), src_dst_pairs, pr.size() * sizeof(int64_t), hipMemcpyDefault, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return fail(PA_ERR_HIP, "copy_blocks: debug copy failed");
    std::unordered_set<int64_t> dsts, srcs;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int64_t s = pr[2 * i], d = pr[2 * i + 1];
      if (s < 0 || s >= desc->num_blocks || d < 0 || d >= desc->num_blocks)
        return fail(PA_ERR_INVALID, "copy_blocks: pair %d = (%lld, %lld) outside the pool", i, (long long)s,
                    (long long)d);
      if (!dsts.insert(d).second) return fail(PA_ERR_INVALID, "copy_blocks: destination %lld repeated", (long long)d);
      srcs.insert(s);
    }
    for (int64_t d : dsts)
      if (srcs.count(d)) return fail(PA_ERR_INVALID, "copy_blocks: block %lld is both source and destination",
                                     (long long)d);
  }
  const int eb = desc->dtype == PA_F32 ? 4 : 2;
  const int64_t block_vecs = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * desc->head_dim * eb / 16;
  const int64_t per_wg = static_cast<int64_t>(kCopyThreads) * kCopyVecsPerThread;
  const int64_t slices = (block_vecs + per_wg - 1) / per_wg;
  if (slices > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "copy_blocks: block too large");
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(slices), num_pairs, 2), dim3(kCopyThreads), 0,
                     stream, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), src_dst_pairs, block_vecs,
                     static_cast<int64_t>(desc->num_blocks));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "copy_blocks: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_stage_copy(void* dst, const void* src, size_t bytes, void* stream_) {
  clear_error();
  if (bytes == 0) return PA_OK;
  if (!dst || !src) return fail(PA_ERR_INVALID, "pa_stage_copy: NULL pointer");
  if (!aligned16(dst) || !aligned16(src) || bytes % 16 != 0)
    return fail(PA_ERR_INVALID, "pa_stage_copy: pointers and size must be multiples of 16 bytes");
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t want = (n + kCopyThreads - 1) / kCopyThreads;
  const int grid = static_cast<int>(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(stage_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream_),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_stage_copy: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
